// Prefill-side kernel (M > 16): C[M,N] = A[M,K] x W[N,K]^T with INT8
// activations and 4-bit (or 2-bit ternary, or INT8) weights on the CDNA4 INT8
// matrix cores, and FP8 E4M3 x FP8 E4M3 on the FP8 matrix cores
// (v_mfma_f32_16x16x128_f8f6f4, float32 sums).
//
// Dataflow (INT4 quantization page, Part 1 step 3, mapped to gfx950): for each
// k tile, a block copies its activation tile (BM x TILE_K int8) and its
// prepacked weight tiles (BN/16 x 1 KiB, still 4-bit) from global memory into
// one of two LDS buffers while the matrix cores work on the other buffer.
// Each wave reads its fragments from LDS, widens the weight nibbles (crumbs)
// to int8 in registers (values 16*q, or 64*c, so the sign comes for free),
// and issues v_mfma_i32_16x16x64_i8. The INT32 accumulators are exact; the
// epilogue shifts out the 2^4 (2^6) factor and applies
// w_scale * a_scale (+ bias) (INT4 page, Part 1 step 4) before the store.
//
// Block: 2*WM waves in a WM (m) x 2 (n) grid, block tile BM = 64*WM rows x
// BN = 16 * NTILES columns, wave tile 64 x 8*NTILES. WM = 2 runs two blocks
// per CU; WM = 4 runs one 512-thread block per CU, whose two waves per SIMD
// meet at the same barrier every k tile (two independent blocks drift apart:
// the hardware favours the older one, and the younger then finishes alone
// with one wave per SIMD, too few to keep the matrix core busy).
// Blocks are mapped so that each of the 8 XCDs works on a contiguous range of
// weight columns (its slice of W stays in that XCD's L2 while all m blocks
// pass over it).
#pragma once

#include "gemv.hpp"

namespace w4 {

template <int KIND>
struct GemmTraits {
  // weight tiles per n tile per stage: FP8 stages two 64-k tiles, the 128 k
  // of one v_mfma_f32_16x16x128_f8f6f4; every other kind one tile
  static constexpr int WT = KIND == KIND_F8F8 ? 2 : 1;
  static constexpr int TILE_K = KindTraits<KIND>::TILE_K * WT;  // k per stage
  static constexpr int KSTEPS = TILE_K / 64;               // MFMA k steps per lane quarter
  static constexpr int ROW_CHUNKS = TILE_K / 16;           // 16-byte chunks per staged A row
  using Acc = typename std::conditional<KIND == KIND_F8F8, f4, i4>::type;
};

// Physical 16-byte chunk of logical chunk c in staged A row `row`: an XOR
// swizzle that spreads the 16 rows of a fragment read over the LDS banks
// (64-byte rows: four rows share a 256-byte bank line, so the swizzle uses
// row>>2; 128-byte rows alternate between two halves, so it uses row>>1;
// 256-byte rows all start on bank 0, so it uses row itself). On gfx950 a
// 16-byte read in this layout still costs 4 bank-conflict cycles (rocprofv3
// SQ_LDS_BANK_CONFLICT on a probe); a chunk-major layout that has none
// ([row / 16][chunk][row % 16]) needs 16-row x 64-byte direct loads instead of
// 8-row x 128-byte ones and was measured slower (same box, tuner, 100 calls:
// W4A8 256 x 352 at M=2048 N=11008 K=4096 +2%, W8A8 128 x 128 +10%).
template <int KIND>
__device__ __forceinline__ int a_chunk(int row, int c) {
  if constexpr (GemmTraits<KIND>::ROW_CHUNKS == 4) return c ^ ((row >> 2) & 3);
  else if constexpr (GemmTraits<KIND>::ROW_CHUNKS == 8) return c ^ ((row >> 1) & 7);
  else return c ^ (row & 15);
}

template <int KIND, int NTILES, int WM>
struct GemmShape {
  using G = GemmTraits<KIND>;
  static_assert(WM == 2 || WM == 4, "128- or 256-row blocks");
  static constexpr int WAVES = 2 * WM;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int BM = 64 * WM;
  static constexpr int BLOCKS_PER_CU = 4 / WM;                  // two waves per SIMD
  static constexpr int A_BYTES = BM * G::TILE_K;                // unpadded, XOR-swizzled rows
  static constexpr int A_LOADS = A_BYTES / TILE_BYTES;          // 1 KiB wave loads per stage
  static constexpr int W_BYTES = NTILES * G::WT * TILE_BYTES;
  static_assert(NTILES % 2 == 0, "two waves split the block's columns");
  static constexpr int NTW = NTILES / 2;                        // n subtiles per wave
  // LDS rings: two weight stages and two or three activation stages. A third
  // activation stage (the activation tile two k tiles ahead) is used where it
  // fits the CU's 160 KiB beside the rest: the INT8-weight 128 x 128 blocks
  // (M=2048 N=K=4096 on MI355X: 47.5 -> 44.2 us) and the 256 x 352 INT4
  // blocks (M=2048 N=11008 K=4096: 75.6 against 75.3 us without it, means of
  // four alternating runs on one box, i.e. no change); a third weight stage
  // alone was measured no faster there.
  static constexpr int PARAM_BYTES = NTILES * 16 * 6 + BM * 4;
  static constexpr int A_STAGES =
      BLOCKS_PER_CU * (3 * A_BYTES + 2 * W_BYTES + PARAM_BYTES) <= 160 * 1024 ? 3 : 2;
  static constexpr int W_OFF = A_STAGES * A_BYTES;             // weight ring after the activations
  static constexpr int RING = W_OFF + 2 * W_BYTES;
  static constexpr int A_PER_WAVE = A_LOADS / WAVES;            // direct loads per wave
  static constexpr int W_PER_WAVE = (NTILES * G::WT + WAVES - 1) / WAVES;  // last round may be partial
  // fp16 epilogue staging: per wave and pass, 32 rows of 16*NTW columns
  static constexpr int EPI_ROWS = 32;
  static constexpr int EPI_ROW = NTW * 32 + 16;                 // padded row bytes
  static constexpr int EPI = WAVES * EPI_ROWS * EPI_ROW;
  // the block's column scales (f32) and biases (f16), and its row scales
  // (f32), sit in LDS behind the stages when the blocks of a CU still fit its
  // 160 KiB, so that the epilogue neither holds them in registers next to
  // every accumulator nor waits for a load of them after the k loop
  static constexpr int PARAM_OFF = RING > EPI ? RING : EPI;
  static constexpr bool LDS_PARAMS = BLOCKS_PER_CU * (PARAM_OFF + PARAM_BYTES) <= 160 * 1024;
  static constexpr int LDS = PARAM_OFF + (LDS_PARAMS ? PARAM_BYTES : 0);
  static_assert(BLOCKS_PER_CU * LDS <= 160 * 1024, "LDS exceeds the CU");
  // the split-K finish holds every accumulator next to a batch of the other
  // splits' sums; wider blocks would spill, so they only run with ksplit == 1
  static constexpr bool SPLIT_OK = NTILES <= 8;
};

struct GemmGrid {
  int mblocks, nblocks, tiles, ksplit, kts, per_xcd;
};

// unpack one 16-byte weight fragment into KSTEPS int8 MFMA operands
template <int KIND>
__device__ __forceinline__ void unpack_frag(const u4 w, i4 (&bf)[GemmTraits<KIND>::KSTEPS]) {
  if constexpr (KIND == KIND_W8A8) {
    bf[0] = __builtin_bit_cast(i4, w);               // INT8 weights are the operand
  } else if constexpr (KIND == KIND_W4A8) {
    bf[0] = unpack_w4_i8(w[0], w[1]);
    bf[1] = unpack_w4_i8(w[2], w[3]);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) bf[j] = unpack_w2_i8(w[j]);
  }
}

// Epilogue of one accumulator fragment: 4 consecutive output columns n..n+3
// of row m (operands are swapped in the MFMA so a lane owns a column run).
// ws/bias hold the 4 columns' weight scales and biases, sa the row's scale.
template <int KIND, int OUT, bool BIAS, typename V>
__device__ __forceinline__ void gemm_store4(const MMParams& p, int m, int n, const V v,
                                            const f4 ws, const f4 bias, float sa, bool vec_ok) {
  constexpr int SH = KindTraits<KIND>::SHIFT;
  if (m >= p.M || n >= p.N) return;
  const bool full = vec_ok && n + 3 < p.N;
  if constexpr (OUT == W4_OUT_I32 && KIND != KIND_F8F8) {
    int32_t* c = reinterpret_cast<int32_t*>(p.C) + (size_t)m * p.N + n;
    const i4 q = i4{v[0] >> SH, v[1] >> SH, v[2] >> SH, v[3] >> SH};
    if (full) {
      *reinterpret_cast<i4*>(c) = q;
    } else {
      for (int e = 0; e < 4 && n + e < p.N; ++e) c[e] = q[e];
    }
  } else {
    float o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (KIND == KIND_F8F8) o[e] = v[e] * ws[e] * sa;
      else o[e] = (float)(v[e] >> SH) * ws[e] * sa;
      if constexpr (BIAS && OUT == W4_OUT_F16) o[e] += bias[e];
    }
    if constexpr (OUT == W4_OUT_I8 && KIND != KIND_F8F8) {
      // re-quantized for a following INT8 layer, the code decided in float32
      // as the decode kernel decides it
      int8_t* c = reinterpret_cast<int8_t*>(p.C) + (size_t)m * p.N + n;
      for (int e = 0; e < 4 && n + e < p.N; ++e)
        c[e] = (int8_t)sym_code_div(o[e], p.out_scale[0], 127.f);
    } else if constexpr (OUT == W4_OUT_F32) {
      float* c = reinterpret_cast<float*>(p.C) + (size_t)m * p.N + n;
      if (full) {
        *reinterpret_cast<f4*>(c) = f4{o[0], o[1], o[2], o[3]};
      } else {
        for (int e = 0; e < 4 && n + e < p.N; ++e) c[e] = o[e];
      }
    } else {
      uint16_t* c = reinterpret_cast<uint16_t*>(p.C) + (size_t)m * p.N + n;
      if (full) {
        *reinterpret_cast<u2*>(c) = u2{(uint32_t)f2h(o[0]) | ((uint32_t)f2h(o[1]) << 16),
                                       (uint32_t)f2h(o[2]) | ((uint32_t)f2h(o[3]) << 16)};
      } else {
        for (int e = 0; e < 4 && n + e < p.N; ++e) c[e] = f2h(o[e]);
      }
    }
  }
}

// Column scales/biases of the 4 columns starting at n (clamped reads).
template <int KIND, int OUT, bool BIAS>
__device__ __forceinline__ void gemm_col_params(const MMParams& p, int n, f4& ws, f4& bias) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int ne = min(n + e, p.N - 1);
    if constexpr (OUT != W4_OUT_I32) ws[e] = KIND == KIND_W2A8 ? h2f(p.w_scale16[0]) : p.w_scale[ne];
    if constexpr (BIAS && OUT == W4_OUT_F16) bias[e] = h2f(p.bias[ne]);
  }
}

template <int KIND, int NTILES, int WM, int OUT, bool BIAS>
__device__ __forceinline__ void gemm_tile(const MMParams& p, const GemmGrid& gg) {
  using G = GemmTraits<KIND>;
  using S = GemmShape<KIND, NTILES, WM>;
  static_assert(S::THREADS == 128 * WM, "launch bounds");
  constexpr int TK = G::TILE_K;
  constexpr int J = G::KSTEPS;
  constexpr int NTW = S::NTW;
  constexpr int RC = G::ROW_CHUNKS;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  // ---- block -> (m block, n block, k split) -------------------------------
  // Each XCD (blocks id, id + 8, ...) takes a contiguous run of the tile
  // order, which is n-major within each half of the m blocks: at M=2048,
  // N=11008 (8 x 32 tiles) an XCD covers 4 m blocks x 8 n blocks, so its L2
  // pulls in half of A and a quarter of W (78.6 MB from memory in all, against
  // 90 MB when an XCD held all 8 m blocks of 4 n blocks).
  const int id = blockIdx.x;
  const int xcd = id & 7, local = id >> 3;
  const int tix = xcd * gg.per_xcd + local;
  if (local >= gg.per_xcd || tix >= gg.tiles) return;
  int nb, mb;
  if (gg.mblocks % 2 == 0) {
    const int mh = gg.mblocks / 2;
    const int half = tix / (gg.nblocks * mh);
    const int rem = tix - half * gg.nblocks * mh;
    nb = rem / mh;
    mb = half * mh + (rem - nb * mh);
  } else {
    nb = tix / gg.mblocks;
    mb = tix - nb * gg.mblocks;
  }
  const int kz = blockIdx.y;
  const int KS = (p.KT + G::WT - 1) / G::WT;         // k stages (WT weight tiles each)
  const int kb = kz * gg.kts;
  const int ke = min(KS, kb + gg.kts);
  const int nk = max(0, ke - kb);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % WM, wn = wave / WM;
  const int r = lane & 15, b = lane >> 4;
  const int m0 = mb * S::BM;
  const int t0 = nb * NTILES;                        // first n tile of the block

  const int8_t* A = reinterpret_cast<const int8_t*>(p.A);

  // ---- direct global -> LDS copies of one k tile into stage `st` -----------
  // Each wave instruction fills 1 KiB of LDS (lane l -> bytes 16l..16l+15).
  // Rows past M and k past K read clamped addresses: the weight codes there
  // are zero, so those products vanish, and rows past M are never stored.
  const int lrow = lane / RC, lchunk = lane % RC;    // position within one 1 KiB load
  auto issue_a = [&](int kt, int st) {
    uint8_t* sa = smem + st * S::A_BYTES;
#pragma unroll
    for (int q = 0; q < S::A_PER_WAVE; ++q) {
      const int ld = wave * S::A_PER_WAVE + q;       // 1 KiB load index within the A tile
      const int row = ld * (64 / RC) + lrow;
      const int c = a_chunk<KIND>(row, lchunk);      // logical chunk for this physical slot
      const int gm = min(m0 + row, p.M - 1);
      const int gk = min(kt * TK + 16 * c, p.K - 16);
      __builtin_amdgcn_global_load_lds(A + (size_t)gm * p.K + gk, sa + ld * TILE_BYTES, 16, 0, 0);
    }
  };
  auto issue_w = [&](int kt, int st) {
    uint8_t* sw = smem + S::W_OFF + st * S::W_BYTES;
#pragma unroll
    for (int q = 0; q < S::W_PER_WAVE; ++q) {
      const int tl = q * S::WAVES + wave;            // weight tile slot within the block
      if ((NTILES * G::WT) % S::WAVES != 0 && tl >= NTILES * G::WT) break;  // wave-uniform
      const int t = min(t0 + tl / G::WT, p.NT - 1);
      // the second tile of a stage past the last weight tile (odd tile
      // count) re-reads the last one; its products are dropped in compute
      const int kw = min(kt * G::WT + tl % G::WT, p.KT - 1);
      __builtin_amdgcn_global_load_lds(p.Wt + ((size_t)t * p.KT + kw) * TILE_BYTES + lane * 16,
                                       sw + tl * TILE_BYTES, 16, 0, 0);
    }
  };
  using Acc = typename G::Acc;
  auto compute_f8 = [&](int ast, int wst, int kt, auto& acc) {
    // lane (r, b) holds k = 16 b .. 16 b + 15 of each of the stage's two
    // weight tiles; its A operand is the same k positions of its row (chunks
    // b and 4 + b of the 128-byte staged row), so the 128-k product sums the
    // same terms as the two 64-k halves
    const uint8_t* sa = smem + ast * S::A_BYTES;
    const uint8_t* sw = smem + S::W_OFF + wst * S::W_BYTES;
    const bool hi_live = kt * 2 + 1 < p.KT;          // uniform
    v8i af[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 64 * wm + 16 * i + r;
      const u4 lo = *reinterpret_cast<const u4*>(sa + row * TK + 16 * a_chunk<KIND>(row, b));
      const u4 hi = *reinterpret_cast<const u4*>(sa + row * TK + 16 * a_chunk<KIND>(row, 4 + b));
      af[i] = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                  (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
    const uint8_t* swl = sw + wn * NTW * 2 * TILE_BYTES + lane * 16;
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      const u4 lo = *reinterpret_cast<const u4*>(swl + 2 * t * TILE_BYTES);
      u4 hi = *reinterpret_cast<const u4*>(swl + (2 * t + 1) * TILE_BYTES);
      if (!hi_live) hi = u4{0u, 0u, 0u, 0u};
      const v8i bw = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                         (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
#pragma unroll
      for (int i = 0; i < 4; ++i)   // weights as the row operand: lane owns 4 columns
        acc[i][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bw, af[i], acc[i][t], 0, 0, 0,
                                                                     0, 0, 0);
    }
  };
  auto compute = [&](int ast, int wst, auto& acc) {
    const uint8_t* sa = smem + ast * S::A_BYTES;
    const uint8_t* sw = smem + S::W_OFF + wst * S::W_BYTES;
    i4 af[4][J];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 64 * wm + 16 * i + r;
#pragma unroll
      for (int j = 0; j < J; ++j)
        af[i][j] = *reinterpret_cast<const i4*>(sa + row * TK +
                                                16 * a_chunk<KIND>(row, (RC / 4) * b + j));
    }
    // Software pipeline over the wave's weight fragments: fragment t+2 is in
    // flight from LDS and fragment t+1 is unpacked while the MFMAs of
    // fragment t run.
    const uint8_t* swl = sw + wn * NTW * TILE_BYTES + lane * 16;
    u4 w2 = *reinterpret_cast<const u4*>(swl + (NTW > 1 ? TILE_BYTES : 0));
    i4 bc[J];
    unpack_frag<KIND>(*reinterpret_cast<const u4*>(swl), bc);
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      // Least progress first: the two waves of a SIMD run the same fragment
      // sequence, and a wave lowers its priority as it gets through its
      // fragments, so the one that is behind is issued first and both reach
      // the k-tile barrier together (with equal priority the older wave wins
      // every arbitration, and the younger one finishes the tile alone).
      if (t == 0 || (4 * t) / NTW != (4 * (t - 1)) / NTW) {
        switch ((4 * t) / NTW) {
          case 0: __builtin_amdgcn_s_setprio(3); break;
          case 1: __builtin_amdgcn_s_setprio(2); break;
          case 2: __builtin_amdgcn_s_setprio(1); break;
          default: __builtin_amdgcn_s_setprio(0); break;
        }
      }
      u4 w3 = w2;
      if (t + 2 < NTW) w3 = *reinterpret_cast<const u4*>(swl + (t + 2) * TILE_BYTES);
      i4 bn[J];
      if (t + 1 < NTW) unpack_frag<KIND>(w2, bn);
#pragma unroll
      for (int j = 0; j < J; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)   // weights as the row operand: lane owns 4 columns
          acc[i][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(bc[j], af[i][j], acc[i][t], 0, 0, 0);
      if (t + 1 < NTW) {
#pragma unroll
        for (int j = 0; j < J; ++j) bc[j] = bn[j];
        w2 = w3;
      }
    }
  };

  Acc acc[4][NTW];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int t = 0; t < NTW; ++t) acc[i][t] = Acc{};

  // Rings: weight tile i+1 streams into the other weight stage while tile i
  // is multiplied; the activation tile runs two k tiles ahead where there are
  // three activation stages (A3), else one. The wait at the end of step i
  // leaves only the activation loads of tile i+2 in flight (the youngest this
  // wave issued; every wave issues A_PER_WAVE of them), and the barrier
  // publishes tile i+1 and frees the stages of tile i. The barrier is a bare
  // s_barrier after the LDS wait: __syncthreads() would also wait for every
  // copy in flight.
  constexpr bool A3 = S::A_STAGES == 3;
  if (nk > 0) {
    issue_a(kb, 0);
    issue_w(kb, 0);
  }
  if (A3 && nk > 1) issue_a(kb + 1, 1);
  constexpr bool LP = S::LDS_PARAMS && OUT == W4_OUT_F16;
  float* lws = reinterpret_cast<float*>(smem + S::PARAM_OFF);
  uint16_t* lbias = reinterpret_cast<uint16_t*>(smem + S::PARAM_OFF + NTILES * 16 * 4);
  float* lsa = reinterpret_cast<float*>(smem + S::PARAM_OFF + NTILES * 16 * 6);
  if constexpr (LP) {
#pragma unroll
    for (int c = tid; c < NTILES * 16; c += S::THREADS) {
      const int n = min(t0 * 16 + c, p.N - 1);
      lws[c] = KIND == KIND_W2A8 ? h2f(p.w_scale16[0]) : p.w_scale[n];
      if constexpr (BIAS) lbias[c] = p.bias[n];
    }
#pragma unroll
    for (int c = tid; c < S::BM; c += S::THREADS) lsa[c] = p.a_scale[min(m0 + c, p.M - 1)];
  }
  auto wait_next = [&](bool a_ahead) {              // a_ahead: block-uniform
    if (A3 && a_ahead) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(S::A_PER_WAVE) : "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };
  wait_next(nk > 1);
  int ast = 0;                                       // activation stage of tile i
  for (int i = 0; i < nk; ++i) {
    if (i + 1 < nk) issue_w(kb + i + 1, (i + 1) & 1);
    if constexpr (A3) {
      if (i + 2 < nk) issue_a(kb + i + 2, ast == 0 ? 2 : ast - 1);
    } else {
      if (i + 1 < nk) issue_a(kb + i + 1, (i + 1) & 1);
    }
    if constexpr (KIND == KIND_F8F8) compute_f8(ast, i & 1, kb + i, acc);
    else compute(ast, i & 1, acc);
    wait_next(i + 2 < nk);
    ast = A3 ? (ast == 2 ? 0 : ast + 1) : (ast ^ 1);
  }

  // ---- epilogue: lane owns columns n..n+3 of row m for each fragment -------
  const bool vec_ok = (p.N % 4) == 0;
  const int nbase = (t0 + wn * NTW) * 16 + 4 * b;
  float sav[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    sav[i] = OUT == W4_OUT_I32 ? 0.f
             : LP              ? lsa[64 * wm + 16 * i + r]
                               : p.a_scale[min(m0 + 64 * wm + 16 * i + r, p.M - 1)];
  // ---- split K: exact INT32 partial sums through the workspace; the last
  // block of the tile to arrive adds the other blocks' sums to its own
  // accumulators and runs the epilogue below. Integer sums do not depend on
  // the order of the additions, so the result is bit-identical to one pass.
  // Every block of a tile holds the same outputs in the same registers, so
  // the sums are kept in register order: word pair q of thread tid of split z
  // at ((tile * ksplit + z) * Q + q) * THREADS + tid. A wave instruction then
  // moves 512 contiguous bytes, and rows past M or columns past N need no
  // test (their sums are never stored to C).
  if constexpr (S::SPLIT_OK && KIND != KIND_F8F8) {  // float sums are never split
    if (gg.ksplit > 1) {
      constexpr int Q = 8 * NTW;                     // 64-bit words per thread
      uint32_t* tile_part = reinterpret_cast<uint32_t*>(p.partials) +
                            (size_t)tix * gg.ksplit * Q * S::THREADS * 2;
      auto word = [&](int z, int q) {
        return tile_part + ((size_t)(z * Q + q) * S::THREADS + tid) * 2;
      };
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int t = 0; t < NTW; ++t) {
          const int q = (i * NTW + t) * 2;
          dev_store2(word(kz, q), (uint32_t)acc[i][t][0], (uint32_t)acc[i][t][1]);
          dev_store2(word(kz, q + 1), (uint32_t)acc[i][t][2], (uint32_t)acc[i][t][3]);
        }
      // every wave's stores are complete before thread 0 counts the block in
      __shared__ int last;
      stores_done();
      __syncthreads();
      if (tid == 0) last = dev_arrive(&p.counters[tix]) == (unsigned)(gg.ksplit - 1);
      __syncthreads();
      if (!last) return;
      if (tid == 0) dev_store(&p.counters[tix], 0u); // every split has counted in
      // Add the other splits' sums, 32 words per thread at a time: every load
      // of a batch is issued before any is added, so a batch costs one round
      // trip to the level all XCDs share.
      constexpr int IB = 16 / NTW;                   // fragment rows per batch
      for (int j = 0; j < gg.ksplit - 1; ++j) {
        const int z = j + (j >= kz);                 // the other splits in order
#pragma unroll
        for (int i0 = 0; i0 < 4; i0 += IB) {
          // keeps the compiler from hoisting later batches' loads (and their
          // registers) above this batch's additions
          asm volatile("" ::: "memory");
          uint64_t lv[IB][NTW][2];
#pragma unroll
          for (int ii = 0; ii < IB; ++ii)
#pragma unroll
            for (int t = 0; t < NTW; ++t) {
              const int q = ((i0 + ii) * NTW + t) * 2;
              lv[ii][t][0] = dev_load2(word(z, q));
              lv[ii][t][1] = dev_load2(word(z, q + 1));
            }
#pragma unroll
          for (int ii = 0; ii < IB; ++ii)
#pragma unroll
            for (int t = 0; t < NTW; ++t) {
              i4& a = acc[i0 + ii][t];
              a[0] += (int)(uint32_t)lv[ii][t][0];
              a[1] += (int)(uint32_t)(lv[ii][t][0] >> 32);
              a[2] += (int)(uint32_t)lv[ii][t][1];
              a[3] += (int)(uint32_t)(lv[ii][t][1] >> 32);
            }
        }
      }
    }
  }

  if constexpr (OUT == W4_OUT_F16) {
    if ((p.N % 8) == 0) {
      // Stage the wave's fp16 tile in LDS, 32 rows x 16*NTW columns per pass,
      // then store whole 16-byte row chunks (a lane group writes a contiguous
      // row segment). The k loop ended with a barrier, so the stages are
      // free; each wave only touches its own region, and its LDS accesses
      // complete in order, so the passes need no barrier.
      constexpr int WC = NTW * 16;
      constexpr int RS = S::EPI_ROW;
      constexpr int ER = S::EPI_ROWS;
      constexpr int IP = ER / 16;                    // fragments rows per pass
      uint8_t* cw = smem + wave * ER * RS;
      const int n_w = (t0 + wn * NTW) * 16;          // first column of the wave tile
#pragma unroll
      for (int h = 0; h < 4 / IP; ++h) {
#pragma unroll
        for (int t = 0; t < NTW; ++t) {
          f4 ws = f4{0.f, 0.f, 0.f, 0.f}, bias = f4{0.f, 0.f, 0.f, 0.f};
          if constexpr (LP) {
            const int c = (wn * NTW + t) * 16 + 4 * b;
            ws = *reinterpret_cast<const f4*>(lws + c);
            if constexpr (BIAS) {
              const u2 bb = *reinterpret_cast<const u2*>(lbias + c);
              bias = f4{h2f((uint16_t)bb[0]), h2f((uint16_t)(bb[0] >> 16)), h2f((uint16_t)bb[1]),
                        h2f((uint16_t)(bb[1] >> 16))};
            }
          } else {
            gemm_col_params<KIND, OUT, BIAS>(p, nbase + 16 * t, ws, bias);
          }
#pragma unroll
          for (int ii = 0; ii < IP; ++ii) {
            const int i = h * IP + ii;
            uint32_t hv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              float o;
              if constexpr (KIND == KIND_F8F8) o = acc[i][t][e] * ws[e] * sav[i];
              else o = (float)(acc[i][t][e] >> KindTraits<KIND>::SHIFT) * ws[e] * sav[i];
              if constexpr (BIAS) o += bias[e];
              hv[e] = f2h(o);
            }
            *reinterpret_cast<u2*>(cw + (16 * ii + r) * RS + (16 * t + 4 * b) * 2) =
                u2{hv[0] | (hv[1] << 16), hv[2] | (hv[3] << 16)};
          }
        }
#pragma unroll
        for (int q = 0; q < ER * WC / 8 / 64; ++q) {
          const int c = q * 64 + lane;
          const int row = c / (WC / 8), c8 = c % (WC / 8);
          const u4 v = *reinterpret_cast<const u4*>(cw + row * RS + c8 * 16);
          const int m = m0 + 64 * wm + ER * h + row, n = n_w + 8 * c8;
          if (m < p.M && n < p.N)
            *reinterpret_cast<u4*>(reinterpret_cast<uint16_t*>(p.C) + (size_t)m * p.N + n) = v;
        }
      }
      return;
    }
  }
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    f4 ws = f4{0.f, 0.f, 0.f, 0.f}, bias = f4{0.f, 0.f, 0.f, 0.f};
    gemm_col_params<KIND, OUT, BIAS>(p, nbase + 16 * t, ws, bias);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      gemm_store4<KIND, OUT, BIAS>(p, m0 + 64 * wm + 16 * i + r, nbase + 16 * t, acc[i][t], ws,
                                   bias, sav[i], vec_ok);
  }
}

// The fields the block's first loads depend on come as leading scalar
// arguments, preloaded into SGPRs (see k_gemv).
template <int KIND, int NTILES, int WM, int OUT, bool BIAS>
__global__ __launch_bounds__(128 * WM, 2) void k_gemm(const uint8_t* Wt, const void* A, int M,
                                                      int N, int K, int KT, int mblocks,
                                                      int nblocks, int tiles, int per_xcd,
                                                      int kts, const MMParams pin,
                                                      const GemmGrid gin) {
  MMParams p = pin;
  p.Wt = Wt;
  p.A = A;
  p.M = M;
  p.N = N;
  p.K = K;
  p.KT = KT;
  GemmGrid gg = gin;
  gg.mblocks = mblocks;
  gg.nblocks = nblocks;
  gg.tiles = tiles;
  gg.per_xcd = per_xcd;
  gg.kts = kts;
  gemm_tile<KIND, NTILES, WM, OUT, BIAS>(p, gg);
}

// ---------------------------------------------------------------------------
// planning (host)
// ---------------------------------------------------------------------------
constexpr int GEMM_CUS = 256;

struct GemmCfg {
  int ntiles, wm;
  int ks = 0;       // requested k split (0: chosen from the tile count)
};

inline int gemm_tiles(int M, int N, GemmCfg c) {
  return ceil_div(M, 64 * c.wm) * ceil_div(ceil_div(N, TILE_N), c.ntiles);
}

// Block shape per product. 2-bit weights unpack into twice the registers and
// stay at 128 x 128. For W4A8 each candidate is costed by the rounds of
// resident blocks it needs times the work of one round on a CU (256 rows x
// 16*ntiles columns in every candidate); the 352-column shapes never split K,
// so they are only candidates where their grid fills most of the chip.
inline GemmCfg gemm_cfg(int kind, int M, int N) {
  if (kind == KIND_W4A16) {
    // fp16 activations (gemm16.hip): 128-row blocks, one per CU, 256 or 384
    // columns on eight waves, whichever needs fewer rounds x columns
    const GemmCfg a{16, 2}, b{24, 2};
    const int ca = ceil_div(gemm_tiles(M, N, a), GEMM_CUS) * a.ntiles;
    const int cb = ceil_div(gemm_tiles(M, N, b), GEMM_CUS) * b.ntiles;
    // on a tie the wider block (more products per activation fragment read:
    // M=2048 N=11008 K=4096 on MI355X, 190.5 against 207.4 us)
    return cb <= ca ? b : a;
  }
  if (kind != KIND_W4A8) return GemmCfg{8, 2};       // 2-bit, INT8 and FP8 weights: 128 x 128
  const GemmCfg narrow{16, 2};
  GemmCfg best = narrow;
  int best_cost = ceil_div(gemm_tiles(M, N, narrow), GEMM_CUS * 2) * 16;
  for (const GemmCfg c : {GemmCfg{22, 2}, GemmCfg{22, 4}}) {
    const int tiles = gemm_tiles(M, N, c);
    const int slots = GEMM_CUS * 4 / c.wm;
    if (tiles * 4 < slots * 3) continue;           // under 3/4 of the chip
    const int cost = ceil_div(tiles, slots) * c.ntiles;
    if (cost <= best_cost) best = c, best_cost = cost;
  }
  return best;
}

// The tiled GEMM needs enough block tiles to fill the chip without splitting
// K much; smaller products run on the decode kernel, one block per (16-row
// tile, 16-column tile).
inline bool use_gemm(int kind, int M, int N) {
  if (kind != KIND_W4A8 && kind != KIND_W2A8 && kind != KIND_W8A8 && kind != KIND_W4A16 &&
      kind != KIND_F8F8)
    return false;
  if (M <= 16) return false;
  return gemm_tiles(M, N, gemm_cfg(kind, M, N)) >= 128;
}

inline GemmGrid gemm_grid(int kind, int M, int N, int K, GemmCfg c) {
  const Geometry g = geometry(kind == KIND_W2A8                         ? W4_LAYOUT_W2A8
                              : kind == KIND_W8A8 || kind == KIND_F8F8 ? W4_LAYOUT_W8A8
                                                                       : W4_LAYOUT_W4A8,
                              N, K);
  GemmGrid gg{};
  gg.mblocks = ceil_div(M, 64 * c.wm);
  gg.nblocks = ceil_div(g.NT, c.ntiles);
  gg.tiles = gg.mblocks * gg.nblocks;
  // k stages: one weight tile each, two for FP8
  const int stages = kind == KIND_F8F8 ? ceil_div(g.KT, 2) : g.KT;
  // K is split only for integer sums (exact in any order) over blocks of up
  // to 8 weight tiles, with one arrival counter per tile
  int ks = 1;
  if (c.ntiles <= 8 && gg.tiles <= WS_COUNTER_SLOTS && kind != KIND_W4A16 && kind != KIND_F8F8) {
    if (c.ks > 0) ks = c.ks;
    else
      while (gg.tiles * ks < 256 && ceil_div(stages, ks * 2) >= 2) ks *= 2;
  }
  gg.kts = ceil_div(stages, ks);
  gg.ksplit = ceil_div(stages, gg.kts);
  gg.per_xcd = ceil_div(gg.tiles, 8);
  return gg;
}

// counters, then every split's INT32 sums of every block tile
inline size_t gemm_workspace_bytes(int kind, int M, int N, int K, GemmCfg c) {
  const GemmGrid gg = gemm_grid(kind, M, N, K, c);
  if (gg.ksplit == 1) return 0;
  return WS_COUNTERS + (size_t)gg.tiles * gg.ksplit * (64 * c.wm) * (16 * c.ntiles) * sizeof(int32_t);
}

template <int KIND, int NTILES, int WM, int OUT, bool BIAS>
int launch_gemm_o(const MMParams& p, const GemmGrid& gg, hipStream_t stream) {
  using S = GemmShape<KIND, NTILES, WM>;
  const dim3 grid(gg.per_xcd * 8, gg.ksplit);
  allow_smem((const void*)&k_gemm<KIND, NTILES, WM, OUT, BIAS>, S::LDS);
  hipLaunchKernelGGL((k_gemm<KIND, NTILES, WM, OUT, BIAS>), grid, dim3(S::THREADS), S::LDS,
                     stream, p.Wt, p.A, p.M, p.N, p.K, p.KT, gg.mblocks, gg.nblocks, gg.tiles,
                     gg.per_xcd, gg.kts, p, gg);
  return launch_status();
}

template <int KIND, int NTILES, int WM>
int launch_gemm_f(const MMParams& p, const GemmGrid& gg, hipStream_t stream) {
  if constexpr (KIND == KIND_F8F8) {
    // float32 sums: fp16 (with or without bias) or float32 outputs only
    if (p.out_dtype == W4_OUT_F32)
      return launch_gemm_o<KIND, NTILES, WM, W4_OUT_F32, false>(p, gg, stream);
    if (p.out_dtype != W4_OUT_F16) return W4_ERR_ARG;
    if (p.bias) return launch_gemm_o<KIND, NTILES, WM, W4_OUT_F16, true>(p, gg, stream);
    return launch_gemm_o<KIND, NTILES, WM, W4_OUT_F16, false>(p, gg, stream);
  } else {
    if constexpr (KIND == KIND_W8A8) {
      if (p.out_dtype == W4_OUT_I8)
        return launch_gemm_o<KIND, NTILES, WM, W4_OUT_I8, false>(p, gg, stream);
    }
    if (p.out_dtype == W4_OUT_I32)
      return launch_gemm_o<KIND, NTILES, WM, W4_OUT_I32, false>(p, gg, stream);
    if (p.out_dtype == W4_OUT_F32)
      return launch_gemm_o<KIND, NTILES, WM, W4_OUT_F32, false>(p, gg, stream);
    if (p.bias) return launch_gemm_o<KIND, NTILES, WM, W4_OUT_F16, true>(p, gg, stream);
    return launch_gemm_o<KIND, NTILES, WM, W4_OUT_F16, false>(p, gg, stream);
  }
}

template <int KIND, int NTILES, int WM>
int launch_gemm_t(MMParams p, const GemmGrid& gg, void* ws, hipStream_t stream) {
  p.counters = reinterpret_cast<unsigned*>(ws);
  p.partials = ws ? reinterpret_cast<uint8_t*>(ws) + WS_COUNTERS : nullptr;
  return launch_gemm_f<KIND, NTILES, WM>(p, gg, stream);
}

// Defined in gemm_launch.hip (a translation unit of its own, so that the
// GEMM instances compile in parallel with the rest of the library).
int launch_gemm_w4a8(const MMParams& p, GemmCfg c, void* ws, hipStream_t stream);
int launch_gemm_w2a8(const MMParams& p, GemmCfg c, void* ws, hipStream_t stream);
int launch_gemm_w8a8(const MMParams& p, GemmCfg c, void* ws, hipStream_t stream);
int launch_gemm_f8f8(const MMParams& p, GemmCfg c, hipStream_t stream);
int launch_gemm_w4a16(const MMParams& p, GemmCfg c, hipStream_t stream);  // gemm16.hip

template <int KIND>
int launch_gemm(const MMParams& p, GemmCfg c, void* ws, hipStream_t stream) {
  if constexpr (KIND == KIND_W4A8) return launch_gemm_w4a8(p, c, ws, stream);
  else if constexpr (KIND == KIND_W2A8) return launch_gemm_w2a8(p, c, ws, stream);
  else if constexpr (KIND == KIND_W8A8) return launch_gemm_w8a8(p, c, ws, stream);
  else if constexpr (KIND == KIND_W4A16) return launch_gemm_w4a16(p, c, stream);
  else if constexpr (KIND == KIND_F8F8) return launch_gemm_f8f8(p, c, stream);
  else return W4_ERR_ARG;
}

}  // namespace w4
