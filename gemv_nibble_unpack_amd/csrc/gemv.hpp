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

enum Kind {
  KIND_W4A8 = 0, KIND_W4A16 = 1, KIND_W2A8 = 2, KIND_W2A16 = 3, KIND_W8A8 = 4, KIND_F8F8 = 5
};

// Kinds whose matrix-core sums are float32 (fp16 or FP8 operands); the others
// sum exactly in int32.
template <int KIND>
__host__ __device__ constexpr bool float_acc() {
  return KIND == KIND_W4A16 || KIND == KIND_W2A16 || KIND == KIND_F8F8;
}

struct MMParams {
  const void* A;               // int8 or FP8 [M,K] (A8, F8) or fp16 [M,K] (A16)
  const float* a_scale;        // [M] (A8, F8)
  const uint8_t* Wt;           // prepacked code section
  const uint16_t* St;          // W4A16 scale section
  const uint8_t* Zt;           // W4A16 zero section
  const float* w_scale;        // W4A8, W8A8, F8F8 per-row scales [N]
  const uint16_t* w_scale16;   // W2A8 per-tensor scale [1]
  const uint16_t* bias;        // [N] or NULL
  const float* out_scale;      // [1], W4_OUT_I8 only
  void* C;
  int out_dtype;
  int M, N, K, NT, KT, KQ;
  int ksplit, kts;             // split-K factor and k tiles per split
  unsigned* counters;          // [mtiles * ngroups]  (split-K only)
  void* partials;              // [mtiles][ksplit][ngroups][TN*256] 4-byte
};

// ---- unpack helpers (word layouts are fixed by prepack) --------------------
// W4A16: one 32-bit word (8 codes) -> 8 fp16 values (q - z), slots in k order.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t b, uint32_t c);

__device__ __forceinline__ h8 unpack_w4_f16(uint32_t w, h2 zlo, h2 zhi) {
  const uint32_t w8 = w >> 8;
  const h2 p0 = __builtin_bit_cast(h2, and_or(w, 0x000F000Fu, 0x64006400u));    // 1024+q
  const h2 p1 = __builtin_bit_cast(h2, and_or(w, 0x00F000F0u, 0x64006400u));    // 1024+16q
  const h2 p2 = __builtin_bit_cast(h2, and_or(w8, 0x000F000Fu, 0x64006400u));
  const h2 p3 = __builtin_bit_cast(h2, and_or(w8, 0x00F000F0u, 0x64006400u));
  const h2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  const h2 d0 = p0 + zlo;                                       // q - z
  const h2 d1 = __builtin_elementwise_fma(p1, sixteenth, zhi);  // 64+q-(64+z)
  const h2 d2 = p2 + zlo;
  const h2 d3 = __builtin_elementwise_fma(p3, sixteenth, zhi);
  return h8{d0[0], d0[1], d1[0], d1[1], d2[0], d2[1], d3[0], d3[1]};
}

// W4A16, one activation row: one word (8 codes) -> 8 fp16 values with no
// arithmetic: 1024 + q in slots 0, 1, 4, 5 (codes in bits 0..3 of a half) and
// 1024 + 16q in slots 2, 3, 6, 7 (bits 4..7). The staged activations at slots
// 2, 3, 6, 7 are pre-divided by 16, so every product is a*(1024+q) or
// (a/16)*(1024+16q) = 64a + aq; the offsets and the zero point are removed
// per group after the products (see k_gemv, M1).
__device__ __forceinline__ h8 unpack_w4_off(uint32_t w) {
  const uint32_t w8 = w >> 8;
  const u4 v = u4{and_or(w, 0x000F000Fu, 0x64006400u), and_or(w, 0x00F000F0u, 0x64006400u),
                  and_or(w8, 0x000F000Fu, 0x64006400u), and_or(w8, 0x00F000F0u, 0x64006400u)};
  return __builtin_bit_cast(h8, v);
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

// W2A16: the same word (byte j holds k_j, k_{j+4}, k_{j+8}, k_{j+12} as
// two's-complement crumbs) -> two fp16 MFMA operands, k 0..7 and 8..15.
// Bytes are reordered to (b0, b2, b1, b3) so that one mask takes the crumbs
// of k and k+1 into the two halves; flipping each crumb's high bit turns the
// code c into c + 2 in [0, 3]; the 0x6400 exponent makes the half 1024 + c + 2,
// and one packed subtract of 1026 leaves c exactly.
__device__ __forceinline__ void unpack_w2_f16(uint32_t w, h8& lo, h8& hi) {
  const uint32_t v = __builtin_amdgcn_perm(w, w, 0x03010200u) ^ 0xAAAAAAAAu;
  const h2 off = {(_Float16)-1026.0f, (_Float16)-1026.0f};
  h2 pr[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    pr[2 * i] = __builtin_bit_cast(h2, and_or(v >> (2 * i), 0x00030003u, 0x64006400u)) + off;
    pr[2 * i + 1] = __builtin_bit_cast(h2, and_or(v >> (2 * i + 8), 0x00030003u, 0x64006400u)) + off;
  }
  lo = h8{pr[0][0], pr[0][1], pr[1][0], pr[1][1], pr[2][0], pr[2][1], pr[3][0], pr[3][1]};
  hi = h8{pr[4][0], pr[4][1], pr[5][0], pr[5][1], pr[6][0], pr[6][1], pr[7][0], pr[7][1]};
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
template <>
struct KindTraits<KIND_W2A16> {
  static constexpr int TILE_K = 256, A_CHUNKS = 8, SHIFT = 0;
};
template <>
struct KindTraits<KIND_W8A8> {
  static constexpr int TILE_K = 64, A_CHUNKS = 1, SHIFT = 0;
};
template <>
struct KindTraits<KIND_F8F8> {  // FP8 bytes in the INT8-weight tile layout
  static constexpr int TILE_K = 64, A_CHUNKS = 1, SHIFT = 0;
};

// Epilogue for one output element.
template <int KIND>
__device__ __forceinline__ void store_out(const MMParams& p, int m, int n, float facc, int iacc,
                                          float sa) {
  if constexpr (KIND == KIND_W4A16 || KIND == KIND_W2A16) {
    float v = KIND == KIND_W2A16 ? facc * h2f(p.w_scale16[0]) : facc;
    if (p.bias) v += h2f(p.bias[n]);
    reinterpret_cast<uint16_t*>(p.C)[(size_t)m * p.N + n] = f2h(v);
  } else if constexpr (KIND == KIND_F8F8) {
    float v = facc * p.w_scale[n] * sa;
    if (p.out_dtype == W4_OUT_F32) {
      reinterpret_cast<float*>(p.C)[(size_t)m * p.N + n] = v;
    } else {
      if (p.bias) v += h2f(p.bias[n]);
      reinterpret_cast<uint16_t*>(p.C)[(size_t)m * p.N + n] = f2h(v);
    }
  } else {
    const int acc = iacc >> KindTraits<KIND>::SHIFT;  // exact: the sum is a multiple of 2^SHIFT
    if (p.out_dtype == W4_OUT_I32) {
      reinterpret_cast<int32_t*>(p.C)[(size_t)m * p.N + n] = acc;
      return;
    }
    const float ws = KIND == KIND_W2A8 ? h2f(p.w_scale16[0]) : p.w_scale[n];
    float v = (float)acc * ws * sa;
    if (p.out_dtype == W4_OUT_I8) {
      // re-quantized for a following INT8 layer, the code decided in float32
      reinterpret_cast<int8_t*>(p.C)[(size_t)m * p.N + n] =
          (int8_t)sym_code_div(v, p.out_scale[0], 127.f);
    } else if (p.out_dtype == W4_OUT_F32) {
      reinterpret_cast<float*>(p.C)[(size_t)m * p.N + n] = v;
    } else {
      if (p.bias) v += h2f(p.bias[n]);
      reinterpret_cast<uint16_t*>(p.C)[(size_t)m * p.N + n] = f2h(v);
    }
  }
}

// v_and_or_b32: (a & b) | c in one VALU op (the compiler splits the
// expression into two ops).
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t b, uint32_t c) {
  uint32_t d;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
  return d;
}

// One weight tile times its activation fragments into the accumulator:
// unpack in registers, then the tile's MFMAs (lane quarter b covers a
// contiguous quarter of the tile's k range in both operands). W4A16 scales
// each 128-k partial by its fp16 group scale; the A8 kinds and W2A16 leave
// their scales to the epilogue.
template <int KIND, typename Acc, int AC>
__device__ __forceinline__ void tile_mma(const u4& w, const u4 (&af)[AC], uint16_t sv, uint8_t zv,
                                         Acc& acc) {
  if constexpr (KIND == KIND_W4A16) {
    const _Float16 z = (_Float16)(float)zv;
    const _Float16 zl = -((_Float16)1024.0f + z);
    const _Float16 zh = -((_Float16)64.0f + z);
    const h2 zlo = {zl, zl}, zhi = {zh, zh};
    f4 part = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const h8 bf = unpack_w4_f16(w[j], zlo, zhi);
      part = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, af[j]), bf, part, 0, 0,
                                                    0);
    }
    const float s = h2f(sv);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = fmaf(part[e], s, acc[e]);
  } else if constexpr (KIND == KIND_W2A16) {
    // fp32 sums of exact fp16 products
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      h8 b0, b1;
      unpack_w2_f16(w[j], b0, b1);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, af[2 * j]), b0, acc, 0,
                                                   0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, af[2 * j + 1]), b1, acc,
                                                   0, 0, 0);
    }
  } else if constexpr (KIND == KIND_W4A8) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const i4 bf = unpack_w4_i8(w[2 * j], w[2 * j + 1]);
      acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i4, af[j]), bf, acc, 0, 0, 0);
    }
  } else if constexpr (KIND == KIND_W8A8) {
    // INT8 weights are the operand as they are
    acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i4, af[0]),
                                                __builtin_bit_cast(i4, w), acc, 0, 0, 0);
  } else if constexpr (KIND == KIND_F8F8) {
    // FP8 bytes as stored: each lane's 16 bytes (the same k positions in both
    // operands) feed two 32-k products, low and high 8 bytes; the products
    // are exact and the matrix core sums them in float32
    const u4 a = af[0];
    const long a0 = __builtin_bit_cast(long, u2{a[0], a[1]});
    const long a1 = __builtin_bit_cast(long, u2{a[2], a[3]});
    const long w0 = __builtin_bit_cast(long, u2{w[0], w[1]});
    const long w1 = __builtin_bit_cast(long, u2{w[2], w[3]});
    acc = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a0, w0, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a1, w1, acc, 0, 0, 0);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const i4 bf = unpack_w2_i8(w[j]);
      acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i4, af[j]), bf, acc, 0, 0, 0);
    }
  }
}

// Activation staging geometry: the block's rows x k range, row-major in LDS
// with the row stride padded by 16 bytes so the 16 lanes of a fragment read
// (one per row) fall on different banks.
template <int KIND>
struct AStage {
  static constexpr int ESZ = KIND == KIND_W4A16 || KIND == KIND_W2A16 ? 2 : 1;  // element bytes
  static constexpr int TILE_ROWB = KindTraits<KIND>::TILE_K * ESZ;  // bytes per row per tile
};

// Grid: x = n tile, y = k split, z = 16-row m tile. Block = WAVES waves.
// Phase 1: (STAGED) every thread issues its APER 16-byte activation loads;
// then each wave issues the weight-tile (and group scale/zero) loads of its
// whole contiguous k run (at most MAXT tiles per pass). Phase 2: (STAGED)
// activations go to LDS, one barrier. Phase 3: tiles are unpacked and
// multiplied in order, each waiting only for its own loads. Without STAGED
// (activation rows too large for LDS) each lane loads its own activation
// fragments from L2 through a ring of RING tiles in flight.
//
// FQ (fused activation quantization, A8 kinds, STAGED only): A holds fp16
// (FQ = 1) or fp32 (FQ = 2) rows instead of int8 codes. Each block computes
// the per-token scale of its rows from the whole row (the same max, the same
// float32 division and the same code decision as quantize_a8, so the codes are
// identical), quantizes its staged k range straight into LDS, and keeps the
// scales for the epilogue. Rows <= 8: the waves split into groups of G waves
// per row; rows > 8: wave w owns rows w and w + 8. Each lane holds up to FQC
// 8-element chunks of its rows, loaded before the weight tiles.
//
// M1 (W4A16, one activation row, wave staging, one pass): the codes go to the
// matrix core as 1024 + q or 1024 + 16q (unpack_w4_off) against activations
// whose slots 2, 3, 6, 7 are pre-divided by 16 when staged. A tile's product
// is then part = 1024*SL + 64*SH + sum(a*q), where SL and SH are the group's
// activation sums over the two slot classes; its contribution is
// s * (part - 1024*SL - 64*SH - z*(SL + SH)) = s * sum(a*(q - z)), with the
// sums formed once per wave from the staged rows. Only the row-0 output of
// each lane is kept.
//
// The fields the first loads depend on come as leading scalar arguments: the
// library is built with kernel-argument preloading, so they arrive in SGPRs
// with the wave instead of through a kernel-argument fetch (a memory round
// trip of a few hundred ns in front of the first weight load); the other
// fields of p are fetched while the weights stream.
template <int KIND, int WAVES, int MAXT, int APER, bool STAGED, int FQ = 0, int FQC = 1,
          bool WST = false, bool M1 = false>
__global__ __launch_bounds__(WAVES * 64) void k_gemv(const uint8_t* Wt, const void* A,
                                                     const uint16_t* St, const uint8_t* Zt, int M,
                                                     int K, int KT, int KQ, int kts,
                                                     const MMParams pin) {
  static_assert(FQ == 0 || (STAGED && (KIND == KIND_W4A8 || KIND == KIND_W2A8) && WAVES == 8),
                "fused quantization");
  static_assert(!WST || (STAGED && FQ == 0), "wave staging");
  static_assert(!M1 || (KIND == KIND_W4A16 && WST), "one-row offset scheme");
  MMParams p = pin;
  p.Wt = Wt;
  p.A = A;
  p.St = St;
  p.Zt = Zt;
  p.M = M;
  p.K = K;
  p.KT = KT;
  p.KQ = KQ;
  p.kts = kts;
  using AS = AStage<KIND>;
  constexpr bool A16 = KIND == KIND_W4A16 || KIND == KIND_W2A16;  // fp16 activations
  constexpr bool GRP = KIND == KIND_W4A16;                         // group scales and zeros
  // K need not be a multiple of the tile's k extent (every kind but W4A16,
  // whose K is a multiple of its 128 group): activation reads past K are
  // clamped into the row and their fragments zeroed
  constexpr bool KTAIL = KIND != KIND_W4A16;
  constexpr int NTHR = WAVES * 64;
  constexpr bool FACC = float_acc<KIND>();                        // float32 sums
  typedef typename std::conditional<FACC, f4, i4>::type Acc;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15;   // A row within the m tile / W row within the n tile
  const int b = lane >> 4;   // k quarter of a tile
  // block id -> (n tile, m tile): ids xcd, xcd+8, xcd+16, ... (one XCD) walk
  // the m tiles of one n tile before moving on, so its weights stay in L2
  const int mtiles = (p.M + 15) / 16;
  int tile, mtile;
  if (mtiles == 1) {
    tile = blockIdx.x;
    mtile = 0;
  } else {
    const int id = blockIdx.x, xcd = id & 7, local = id >> 3;
    const int per_xcd = (int)(gridDim.x >> 3);        // grid is a multiple of 8 here
    const int seq = xcd * per_xcd + local;           // position in the XCD's run
    tile = seq / mtiles;
    mtile = seq - tile * mtiles;
    if (local >= per_xcd || tile >= p.NT) return;
  }
  const int rows = min(16, p.M - mtile * 16);
  const int kb = blockIdx.y * p.kts;
  const int ke = min(p.KT, kb + p.kts);
  // W4A16 runs start on an even tile (kts is even), so the scales and zeros
  // of a wave's tiles come in whole quads of groups, one load each
  const int per = GRP ? ((ke - kb + 1) / 2 + WAVES - 1) / WAVES * 2 : (ke - kb + WAVES - 1) / WAVES;
  const int wb = kb + wave * per;
  const int nt = max(0, min(ke, wb + per) - wb);     // tiles of this wave (uniform)

  // ---- phase 0 (FQ): whole activation rows, 8 elements per chunk ----------
  constexpr int FESZ = FQ == 2 ? 4 : 2;              // input element bytes
  constexpr int FU4 = FESZ / 2;                      // u4 loads per chunk
  __shared__ float fq_part[WAVES * 2];               // per wave, per owned row: partial max
  __shared__ float fq_s[16];                         // per row: the activation scale
  u4 fqr[FQ ? FQC * FU4 : 1];
  const int rpw = rows > 8 ? 2 : 1;                  // rows per wave
  const int fq_g = rows > 8 ? 1 : rows > 4 ? 1 : rows > 2 ? 2 : rows > 1 ? 4 : 8;  // waves per row
  const int cpk = p.K / 8;                           // chunks per row
  const int fq_per = (cpk + 64 * fq_g - 1) / (64 * fq_g);  // chunk slots per lane per row
  auto fq_slot = [&](int sl, int& row, int& col) {   // slot -> (row, chunk) or row = -1
    const int rr = sl / fq_per, j = sl - rr * fq_per;
    row = rows > 8 ? wave + 8 * rr : wave / fq_g;
    col = (wave % fq_g) * 64 + lane + 64 * fq_g * j;
    if (rr >= rpw || row >= rows || col >= cpk) row = -1;
  };
  if constexpr (FQ != 0) {
    const uint8_t* Ab0 = reinterpret_cast<const uint8_t*>(p.A);
#pragma unroll
    for (int sl = 0; sl < FQC; ++sl) {
      int row, col;
      fq_slot(sl, row, col);
      // dead slots re-read chunk 0 of row 0 (unconditional loads, exact waits)
      const size_t off = row < 0 ? (size_t)mtile * 16 * p.K * FESZ
                                 : ((size_t)(mtile * 16 + row) * p.K + (size_t)col * 8) * FESZ;
#pragma unroll
      for (int h = 0; h < FU4; ++h) fqr[sl * FU4 + h] = *reinterpret_cast<const u4*>(Ab0 + off + 16 * h);
    }
  }

  // ---- phase 1a: activation loads (row-major chunks of 16 bytes) ----------
  const int rowb = (ke - kb) * AS::TILE_ROWB;        // bytes of one staged row
  const int cpr = rowb / 16;
  const int total = rows * cpr;
  const int sstride = rowb + 16;
  const uint8_t* Ab = reinterpret_cast<const uint8_t*>(p.A);
  const size_t arow_bytes = (size_t)p.K * AS::ESZ;
  const size_t kbyte0 = (size_t)kb * AS::TILE_ROWB;
  // WST: each wave stages only its own k range [wb, wb + per) of the block's
  // rows, in a region of its own, and is the only reader of it, so no block
  // barrier stands between a wave's loads and its first products. APER then
  // counts 16-byte loads per lane of the wave.
  const int wrowb = per * AS::TILE_ROWB;             // bytes of one row of the wave's range
  const int wcpr = wrowb / 16;
  const int wtotal = rows * wcpr;
  const int wstride = wrowb + 16;
  const int wreg = WST ? wave * rows * wstride : 0;  // LDS offset of the wave's region
  const size_t wbyte0 = (size_t)wb * AS::TILE_ROWB;
  u4 stage[APER];
  if constexpr (WST) {
#pragma unroll
    for (int i = 0; i < APER; ++i) {
      const int c = min(lane + i * 64, wtotal - 1);
      const int row = small_div(c, wcpr), col = c - row * wcpr;
      // past the wave's run or past K: clamp into the row, zeroed below
      const size_t off = min(wbyte0 + (size_t)col * 16, arow_bytes - 16);
      stage[i] = *reinterpret_cast<const u4*>(Ab + (size_t)(mtile * 16 + row) * arow_bytes + off);
    }
  } else {
#pragma unroll
    for (int i = 0; i < (STAGED && FQ == 0 ? APER : 0); ++i) {
      const int c = min(tid + i * NTHR, total - 1);
      const int row = small_div(c, cpr), col = c - row * cpr;
      size_t off = kbyte0 + (size_t)col * 16;
      if constexpr (KTAIL) off = min(off, arow_bytes - 16);  // k tail: clamp, zeroed below
      stage[i] = *reinterpret_cast<const u4*>(Ab + (size_t)(mtile * 16 + row) * arow_bytes + off);
    }
  }

  // Loads complete in issue order, so the activation loads (needed before any
  // product) must be issued before the weight tiles. The empty asm statement
  // with a memory clobber keeps the compiler from moving them after (left
  // alone it may, and the wait before their LDS write then waits for every
  // weight tile too).
  asm volatile("" ::: "memory");

  // ---- phase 1b: this wave's weight tiles --------------------------------
  Acc acc = Acc{};
  // M1: per staged chunk, the float32 activation sums over its two slot
  // classes; then per tile of the run, the offset 1024*SL + 64*SH and SL + SH
  float m1_sl[M1 ? APER : 1], m1_sh[M1 ? APER : 1], m1_off[M1 ? MAXT : 1], m1_sum[M1 ? MAXT : 1];
#pragma unroll
  for (int i = 0; i < (M1 ? APER : 1); ++i) m1_sl[i] = m1_sh[i] = 0.f;
  for (int pass = 0; pass * MAXT < max(nt, 1); ++pass) {
    const int pb = wb + pass * MAXT;
    const int pn = min(MAXT, nt - pass * MAXT);      // tiles in this pass (uniform)
    u4 wv[MAXT];
    // W4A16: the pass starts on an even tile, so its tiles' group scales and
    // zeros lie in the NQ quads from pb / 4 on: one 8-byte scale load and one
    // 4-byte zero load per quad (a quad past the row's last reads the last).
    // Quad q is loaded just before tile 4q - 2, in time for a pass that starts
    // mid-quad (tiles 4q - 2 ..) as well as for one that starts on a quad.
    // A pass covers group positions 0 .. MAXT + 1 (mid-quad: shifted by 2).
    constexpr int NQ = GRP ? (MAXT >= 4 ? (MAXT + 1) / 4 + 1 : 1) : 1;
    uint64_t sq[NQ];
    uint32_t zq[NQ];
    auto quad_load = [&](int q) {
      const int qq = min((pb >> 2) + q, p.KQ - 1);
      const size_t mq = (((size_t)tile * p.KQ + qq) * TILE_N + r) * 4;
      if (MAXT >= 4 && MAXT % 4 == 0 && q == NQ - 1) {
        // only groups 0 and 1 of the last quad can be used: loading no more
        // leaves no dead register half that the allocator could reuse while
        // the load is in flight (which would force a wait for it)
        sq[q] = *reinterpret_cast<const uint32_t*>(p.St + mq);
        zq[q] = *reinterpret_cast<const uint16_t*>(p.Zt + mq);
      } else {
        sq[q] = *reinterpret_cast<const uint64_t*>(p.St + mq);
        zq[q] = *reinterpret_cast<const uint32_t*>(p.Zt + mq);
      }
    };
    // tile u's scale and zero, taken where they are used, so that the wait
    // for them covers only the loads issued up to their quad
    const bool mid = (pb & 2) != 0;                  // the pass starts mid-quad
    auto scale_of = [&](int u) -> uint16_t {
      if constexpr (GRP) {
        const uint16_t s0 = (uint16_t)(sq[u >> 2] >> (16 * (u & 3)));
        const uint16_t s1 = (uint16_t)(sq[(u + 2) >> 2] >> (16 * ((u + 2) & 3)));
        return mid ? s1 : s0;
      } else {
        return 0;
      }
    };
    auto zero_of = [&](int u) -> uint8_t {
      if constexpr (GRP) {
        const uint8_t z0 = (uint8_t)(zq[u >> 2] >> (8 * (u & 3)));
        const uint8_t z1 = (uint8_t)(zq[(u + 2) >> 2] >> (8 * ((u + 2) & 3)));
        return mid ? z1 : z0;
      } else {
        return 0;
      }
    };
    // Unconditional loads keep the wait counts exact: slots past the run
    // read tile 0 (a fixed, cache-resident address) and are skipped below.
#pragma unroll
    for (int u = 0; u < MAXT; ++u) {
      if constexpr (GRP) {
#pragma unroll
        for (int q = 0; q < NQ; ++q)
          if (u == (q == 0 ? 0 : 4 * q - 2)) quad_load(q);
      }
      const bool live = u < pn;
      const int kt = pb + u;
      const size_t ti = live ? (size_t)tile * p.KT + kt : 0;
      const u4* wp = reinterpret_cast<const u4*>(p.Wt + ti * TILE_BYTES + lane * 16);
      // streamed once unless several m tiles share the weight tile through L2
      wv[u] = mtiles == 1 ? __builtin_nontemporal_load(wp) : *wp;
    }

    // ---- activation fragments straight from L2 (not STAGED) --------------
    constexpr int RING = 4;
    constexpr int AC = KindTraits<KIND>::A_CHUNKS;
    u4 ring[STAGED ? 1 : RING][AC];
    const size_t arow_g = (size_t)min(mtile * 16 + r, p.M - 1) * arow_bytes;
    auto aload = [&](int u, u4 (&dst)[AC]) {
      // past the run (or for a wave without tiles) re-read a valid tile
      const int kt = min(max(pb + min(u, pn - 1), 0), p.KT - 1);
      const size_t base = (size_t)kt * AS::TILE_ROWB + (AS::TILE_ROWB / 4) * b;
#pragma unroll
      for (int j = 0; j < AC; ++j) {
        size_t off = base + 16 * j;
        if constexpr (KTAIL) off = min(off, arow_bytes - 16);
        dst[j] = *reinterpret_cast<const u4*>(Ab + arow_g + off);
      }
    };
    if constexpr (!STAGED) {
#pragma unroll
      for (int u = 0; u < RING; ++u) aload(u, ring[u]);
    }

    // ---- phase 2: activations to LDS (first pass only) -------------------
    if (FQ != 0 && pass == 0) {
      auto chunk = [&](int sl, float (&x)[8]) {
        if constexpr (FQ == 1) {
          const h8 hv = __builtin_bit_cast(h8, fqr[sl]);
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = (float)hv[e];
        } else {
          // whole-vector casts (a bit cast of one ext-vector element reads
          // element 0 with this compiler)
          const f4 a0 = __builtin_bit_cast(f4, fqr[sl * 2]);
          const f4 a1 = __builtin_bit_cast(f4, fqr[sl * 2 + 1]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            x[e] = a0[e];
            x[4 + e] = a1[e];
          }
        }
      };
      // per-wave maxima of the owned rows, then the row maxima across the group
      float mx[2] = {0.f, 0.f};
#pragma unroll
      for (int sl = 0; sl < FQC; ++sl) {
        int row, col;
        fq_slot(sl, row, col);
        if (row < 0) continue;
        float x[8];
        chunk(sl, x);
        float m = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(x[e]));
        const int rr = sl / fq_per;
        mx[rr] = fmaxf(mx[rr], m);
      }
      mx[0] = wave_max(mx[0]);
      mx[1] = wave_max(mx[1]);
      if (lane == 0) {
        fq_part[wave * 2] = mx[0];
        fq_part[wave * 2 + 1] = mx[1];
      }
      __syncthreads();
      auto row_scale = [&](int row) {
        float m = 0.f;
        if (rows > 8) {
          m = fq_part[(row & 7) * 2 + (row >> 3)];
        } else {
          for (int g = 0; g < fq_g; ++g) m = fmaxf(m, fq_part[(row * fq_g + g) * 2]);
        }
        return m / 127.0f;
      };
      if (tid < rows) fq_s[tid] = row_scale(tid);
      // quantize this block's staged k range into LDS
      const int k0 = kb * AS::TILE_ROWB;                 // int8: one byte per element
      const int k1 = min(ke * AS::TILE_ROWB, p.K);
#pragma unroll
      for (int sl = 0; sl < FQC; ++sl) {
        int row, col;
        fq_slot(sl, row, col);
        if (row < 0 || 8 * col < k0 || 8 * col >= k1) continue;
        const float sa = row_scale(row);
        const float rs = sa > 0.f ? 1.0f / sa : 0.f;
        float x[8];
        chunk(sl, x);
        uint32_t lo = 0, hi = 0;
        auto put = [&](int e, int q) {
          const uint32_t bq = (uint32_t)(q & 0xFF);
          if (e < 4) lo |= bq << (8 * e);
          else hi |= bq << (8 * (e - 4));
        };
        if (__builtin_expect(!(rs <= 0x1.fffffep127f), 0)) {  // 1 / sa overflowed
#pragma unroll
          for (int e = 0; e < 8; ++e) put(e, sym_code_div(x[e], sa, 127.f));
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) put(e, sym_code_rcp(x[e], sa, rs, 127.f));
        }
        *reinterpret_cast<u2*>(smem + row * sstride + (8 * col - k0)) = u2{lo, hi};
      }
      // k tail past K inside the last staged tile contributes zero
      const int tail = kb * AS::TILE_ROWB + rowb - k1;   // bytes, a multiple of 16
      for (int c = tid; c < rows * (tail / 16); c += NTHR) {
        const int row = c / (tail / 16), col = c - row * (tail / 16);
        *reinterpret_cast<u4*>(smem + row * sstride + (k1 - k0) + 16 * col) = u4{0u, 0u, 0u, 0u};
      }
      __syncthreads();
    } else if (WST && pass == 0) {
      // a wave's LDS accesses complete in issue order: its reads below see
      // these writes without a barrier
#pragma unroll
      for (int i = 0; i < APER; ++i) {
        const int c = lane + i * 64;
        if (c < wtotal) {
          const int row = small_div(c, wcpr), col = c - row * wcpr;
          u4 v = stage[i];
          if (col * 16 >= nt * AS::TILE_ROWB || wbyte0 + (size_t)col * 16 >= arow_bytes)
            v = u4{0u, 0u, 0u, 0u};
          if constexpr (M1) {
            // this chunk's sums over slots 0, 1, 4, 5 (SL) and 2, 3, 6, 7 (SH)
            // in float32, then slots 2, 3, 6, 7 divided by 16 (exact)
            const uint32_t e0 = v[0], e1 = v[1], e2 = v[2], e3 = v[3];
            const h2 one = {(_Float16)1.0f, (_Float16)1.0f};
            const h2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
            const h2 x0 = __builtin_bit_cast(h2, e0), x1 = __builtin_bit_cast(h2, e1);
            const h2 x2 = __builtin_bit_cast(h2, e2), x3 = __builtin_bit_cast(h2, e3);
            m1_sl[i] = __builtin_amdgcn_fdot2(x0, one, __builtin_amdgcn_fdot2(x2, one, 0.f, false),
                                              false);
            m1_sh[i] = __builtin_amdgcn_fdot2(x1, one, __builtin_amdgcn_fdot2(x3, one, 0.f, false),
                                              false);
            v[1] = __builtin_bit_cast(uint32_t, x1 * sixteenth);
            v[3] = __builtin_bit_cast(uint32_t, x3 * sixteenth);
          }
          *reinterpret_cast<u4*>(smem + wreg + row * wstride + col * 16) = v;
        }
      }
    } else if (STAGED && pass == 0) {
#pragma unroll
      for (int i = 0; i < APER; ++i) {
        const int c = tid + i * NTHR;
        if (c < total) {
          const int row = small_div(c, cpr), col = c - row * cpr;
          u4 v = stage[i];
          if constexpr (KTAIL) {
            if (kbyte0 + (size_t)col * 16 >= arow_bytes) v = u4{0u, 0u, 0u, 0u};
          }
          *reinterpret_cast<u4*>(smem + row * sstride + col * 16) = v;
        }
      }
      __syncthreads();
    }

    if constexpr (M1) {
      // sums over each tile's 16 chunks (16 consecutive lanes), then every
      // tile's pair broadcast to the wave: tile kl's chunks are 16*kl..16*kl+15
#pragma unroll
      for (int i = 0; i < APER; ++i) {
        m1_sl[i] = row_sum16(m1_sl[i]);
        m1_sh[i] = row_sum16(m1_sh[i]);
      }
#pragma unroll
      for (int u = 0; u < MAXT; ++u) {
        const int i = u / 4 < APER ? u / 4 : APER - 1;
        const float off = fmaf(1024.f, m1_sl[i], 64.f * m1_sh[i]);
        const float sum = m1_sl[i] + m1_sh[i];
        m1_off[u] = __builtin_bit_cast(
            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, off), 16 * (u & 3)));
        m1_sum[u] = __builtin_bit_cast(
            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sum), 16 * (u & 3)));
      }
    }

    // ---- phase 3: unpack + matrix-core products, tile by tile ------------
    const int aoff = WST ? wreg + min(r, rows - 1) * wstride : min(r, rows - 1) * sstride;
    const uint8_t* arow = smem + aoff;
#pragma unroll
    for (int u = 0; u < MAXT; ++u) {
      u4 af[AC];
      if constexpr (STAGED) {
        if (u >= pn) continue;                       // uniform: tiles past the wave's run
        const int kl = pb + u - (WST ? wb : kb);     // tile index within the staged range
        const u4* src = reinterpret_cast<const u4*>(arow + kl * AS::TILE_ROWB +
                                                    (AS::TILE_ROWB / 4) * b);
#pragma unroll
        for (int j = 0; j < AC; ++j) af[j] = src[j];
      } else {
#pragma unroll
        for (int j = 0; j < AC; ++j) af[j] = ring[u % RING][j];
        aload(u + RING, ring[u % RING]);             // unconditional: keeps wait counts exact
      }
      if (u >= pn) continue;                         // uniform: tiles past the wave's run
      if constexpr (KTAIL && !STAGED) {
        // k tail: fragments past K contribute zero (staged rows are zero-filled)
        const int kt = pb + u;
#pragma unroll
        for (int j = 0; j < AC; ++j)
          if ((size_t)kt * AS::TILE_ROWB + (AS::TILE_ROWB / 4) * b + 16 * j >= arow_bytes)
            af[j] = u4{0u, 0u, 0u, 0u};
      }
      if constexpr (M1) {
        f4 part = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t wj = wv[u][j];
          part = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, af[j]),
                                                        unpack_w4_off(wj), part, 0, 0, 0);
        }
        const float p0 = part[0];
        const float t = fmaf(-(float)zero_of(u), m1_sum[u], p0 - m1_off[u]);
        acc[0] = fmaf(t, h2f(scale_of(u)), acc[0]);
      } else {
        tile_mma<KIND>(wv[u], af, scale_of(u), zero_of(u), acc);
      }
    }
  }

  const int ngroups = p.NT;
  const size_t slot = (size_t)mtile * ngroups + tile;
  auto row_sa = [&](int row) {                       // the row's activation scale (A8 kinds)
    if constexpr (A16) return 0.f;
    else if constexpr (FQ != 0) return fq_s[row];
    else return p.a_scale[mtile * 16 + row];
  };
  constexpr int NOUT = 256;                          // 16 x 16 outputs of the tile

  // ---- cross-wave reduction through LDS (reuses the staging buffer) -----
  // MFMA 16x16 output: lane holds column (lane & 15), rows 4*(lane >> 4) + e.
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);       // [WAVES][16 rows][16 cols]
  if (rows == 1 && p.ksplit == 1) {
    // one row: only row 0 (lanes 0..15, element 0) is an output
    if (lane < 16) {
      const auto v = acc[0];
      red[wave * 16 + lane] = __builtin_bit_cast(float, v);
    }
    __syncthreads();
    const int n = tile * 16 + tid;
    if (tid < 16 && n < p.N) {
      float fs = 0.f;
      int is = 0;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) {
        const float v = red[w * 16 + tid];
        if constexpr (FACC) fs += v;
        else is += __builtin_bit_cast(int, v);
      }
      store_out<KIND>(p, mtile * 16, n, fs, is, row_sa(0));
    }
    return;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    // copy the element to a scalar first: __builtin_bit_cast applied to an
    // ext-vector element reads element 0 with this compiler
    const auto v = acc[e];
    red[(wave * 16 + 4 * b + e) * 16 + r] = __builtin_bit_cast(float, v);
  }
  __syncthreads();

  if (p.ksplit == 1) {
    for (int idx = tid; idx < NOUT; idx += NTHR) {
      const int row = idx >> 4, col = idx & 15;
      const int n = tile * 16 + col;
      if (row >= rows || n >= p.N) continue;
      float fs = 0.f;
      int is = 0;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) {
        const float v = red[(w * 16 + row) * 16 + col];
        if constexpr (FACC) fs += v;
        else is += __builtin_bit_cast(int, v);
      }
      store_out<KIND>(p, mtile * 16 + row, n, fs, is, row_sa(row));
    }
    return;
  }

  // ---- split-K: publish this block's partial, the last block finishes ----
  uint32_t* part = reinterpret_cast<uint32_t*>(p.partials) +
                   ((size_t)mtile * p.ksplit + blockIdx.y) * ngroups * NOUT +
                   (size_t)tile * NOUT;
  for (int idx = tid; idx < NOUT; idx += NTHR) {
    const int row = idx >> 4, col = idx & 15;
    float fs = 0.f;
    int is = 0;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
      const float v = red[(w * 16 + row) * 16 + col];
      if constexpr (FACC) fs += v;
      else is += __builtin_bit_cast(int, v);
    }
    dev_store(&part[idx], FACC ? __builtin_bit_cast(uint32_t, fs) : (uint32_t)is);
  }
  // every wave's partial stores are complete before thread 0 counts the
  // block in; the last block reads the partials at device scope
  __shared__ int last;
  stores_done();
  __syncthreads();
  if (tid == 0) last = dev_arrive(&p.counters[slot]) == (unsigned)(p.ksplit - 1);
  __syncthreads();
  if (!last) return;
  const uint32_t* base = reinterpret_cast<const uint32_t*>(p.partials) +
                         (size_t)mtile * p.ksplit * ngroups * NOUT + (size_t)tile * NOUT;
  for (int idx = tid; idx < NOUT; idx += NTHR) {
    const int row = idx >> 4, col = idx & 15;
    const int n = tile * 16 + col;
    if (row >= rows || n >= p.N) continue;
    float fs = 0.f;
    int is = 0;
    dev_sum<FACC>(base + idx, (size_t)ngroups * NOUT, p.ksplit, fs, is);
    store_out<KIND>(p, mtile * 16 + row, n, fs, is, row_sa(row));
  }
  if (tid == 0) dev_store(&p.counters[slot], 0u);  // leave the workspace zeroed
}

}  // namespace w4
