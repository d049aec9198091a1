// Prefill-side kernel (M > 16): C[M,N] = A[M,K] x W[N,K]^T with INT8
// activations and 4-bit (or 2-bit ternary, or INT8) weights on the CDNA4 INT8
// matrix cores.
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
  static constexpr int TILE_K = KindTraits<KIND>::TILE_K;  // k per stage (one weight tile)
  static constexpr int KSTEPS = TILE_K / 64;               // MFMA k steps per lane quarter
  static constexpr int ROW_CHUNKS = TILE_K / 16;           // 16-byte chunks per staged A row
};

// Physical 16-byte chunk of logical chunk c in staged A row `row`: an XOR
// swizzle that puts the 16 rows of a fragment read on distinct LDS banks
// (64-byte rows: four rows share a 256-byte bank line, so the swizzle uses
// row>>2; 128-byte rows alternate between two halves, so it uses row>>1;
// 256-byte rows all start on bank 0, so it uses row itself).
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
  static constexpr int W_BYTES = NTILES * TILE_BYTES;
  static_assert(NTILES % 2 == 0, "two waves split the block's columns");
  static constexpr int NTW = NTILES / 2;                        // n subtiles per wave
  static constexpr int STAGE = A_BYTES + W_BYTES;
  // LDS stages in the ring (two fit the CU's 160 KiB in every configuration;
  // a third weight stage, fetching the weights two k tiles ahead, was
  // measured no faster on the 256 x 352 blocks and is not used)
  static constexpr int STAGES = 2;
  static constexpr int A_PER_WAVE = A_LOADS / WAVES;            // direct loads per wave
  static constexpr int W_PER_WAVE = (NTILES + WAVES - 1) / WAVES;  // last round may be partial
  // fp16 epilogue staging: per wave and pass, 32 rows of 16*NTW columns
  static constexpr int EPI_ROWS = 32;
  static constexpr int EPI_ROW = NTW * 32 + 16;                 // padded row bytes
  static constexpr int EPI = WAVES * EPI_ROWS * EPI_ROW;
  // the block's column scales (f32) and biases (f16) sit in LDS behind the
  // stages when two blocks still fit a CU's 160 KiB, so that the epilogue
  // does not hold them in registers next to every accumulator
  static constexpr int PARAM_OFF = STAGES * STAGE > EPI ? STAGES * STAGE : EPI;
  static constexpr int PARAM_BYTES = NTILES * 16 * 6;
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
template <int KIND, int OUT, bool BIAS>
__device__ __forceinline__ void gemm_store4(const MMParams& p, int m, int n, const i4 v,
                                            const f4 ws, const f4 bias, float sa, bool vec_ok) {
  constexpr int SH = KindTraits<KIND>::SHIFT;
  if (m >= p.M || n >= p.N) return;
  const bool full = vec_ok && n + 3 < p.N;
  if constexpr (OUT == W4_OUT_I32) {
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
      const int a = v[e] >> SH;
      o[e] = (float)a * ws[e] * sa;
      if constexpr (BIAS && OUT == W4_OUT_F16) o[e] += bias[e];
    }
    if constexpr (OUT == W4_OUT_I8) {
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

// ---------------------------------------------------------------------------
// One-launch fused prefill (FQ = 1: fp16 rows, FQ = 2: float32 rows in
// p.A_in). Every wave of the grid first takes activation rows from a shared
// counter, one at a time, and quantizes each whole row with the per-token
// rule of quantize_a8 (INT4 page, Part 1 step 2: scale = max|a| / 127,
// code = rint(a / scale)), writing the int8 row to p.A and its scale to
// p.a_scale, then counts the row in for its m block. A block then waits until
// its m block's rows are all in before it loads activations. This cannot
// deadlock whatever the number of resident blocks: a block waits only after
// the row counter has run out, i.e. when every row has been claimed by a wave
// that is running and that waits for nothing before it finishes its row. The
// wait is bounded anyway (FQ_SPIN_LIMIT polls) so that no wave can spin for
// ever. The counter is polled with an atomic read-modify-write (dev_count):
// plain loads of it are not guaranteed to see other XCDs' increments. The
// last block to finish leaves the counters zero for the next call.
//
// Visibility across XCDs: the rows and scales are written with device-scope
// (sc1) stores, which pass through to the memory all XCDs share, and a wave
// waits for their completion (vmcnt 0) before it counts the row in with a
// device-scope atomic; the waiting block polls the counter with device-scope
// atomics, executes a device-scope acquire fence (the L2 and L1 invalidation
// the AMDGPU memory model prescribes for an agent-scope acquire on gfx950),
// and reads the rows and scales with device-scope (sc1) loads, the same
// store / wait / count / load sequence as the split-K partial sums.
// ---------------------------------------------------------------------------
constexpr unsigned FQ_SPIN_LIMIT = 1u << 18;    // polls of ~0.5-2 us: under a second

template <int FQ, int BM>
__device__ __forceinline__ void fq_quantize_rows(const MMParams& p) {
  constexpr int ESZ = FQ == 2 ? 4 : 2;               // input element bytes
  constexpr int U = ESZ / 2;                         // 16-byte loads per 8-element chunk
  constexpr int RC = 8;                              // chunks per lane held in registers
  const int lane = threadIdx.x & 63;
  const int K = p.K, nch = K / 8;                    // K % 16 == 0
  const uint8_t* Ain = reinterpret_cast<const uint8_t*>(p.A_in);
  uint32_t* qA = reinterpret_cast<uint32_t*>(const_cast<void*>(p.A));
  uint32_t* sa = reinterpret_cast<uint32_t*>(const_cast<float*>(p.a_scale));
  auto widen = [&](const u4 (&r)[U], float (&x)[8]) {
    if constexpr (FQ == 1) {
      const h8 hv = __builtin_bit_cast(h8, r[0]);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = (float)hv[e];
    } else {
      // whole-vector casts (a bit cast of one ext-vector element reads
      // element 0 with this compiler)
      const f4 a0 = __builtin_bit_cast(f4, r[0]);
      const f4 a1 = __builtin_bit_cast(f4, r[U - 1]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[e] = a0[e];
        x[4 + e] = a1[e];
      }
    }
  };
  auto load = [&](const uint8_t* src, int c, u4 (&r)[U]) {
#pragma unroll
    for (int h = 0; h < U; ++h) r[h] = *reinterpret_cast<const u4*>(src + (size_t)c * 8 * ESZ + 16 * h);
  };
  for (;;) {
    // One claim per wave. The loop holds no lane-dependent branch around a
    // side effect, and the row is wave-uniform in the compiler's eyes (an
    // SGPR from readfirstlane): with the claim and the count-in written as
    // `if (lane == 0) ...` and the row taken from a lane shuffle, the
    // compiler gave the loop per-lane exits in which lane 0 went back for a
    // new claim while the 63 others went round again on a stale row, for
    // ever. Every lane now takes part in the atomics, lane 0 adding 1 and the
    // others 0.
    const unsigned one = lane == 0 ? 1u : 0u;
    const unsigned claim = __hip_atomic_fetch_add(&p.sync[SYNC_NEXT], one, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
    const int row = (int)__builtin_amdgcn_readfirstlane(claim);
    if (row >= p.M) break;                           // uniform
    const uint8_t* src = Ain + (size_t)row * K * ESZ;
    uint32_t* dst = qA + (size_t)row * (K / 4);
    float mx = 0.f, s, rs;
    int sum = 0;
    if (nch <= 64 * RC) {
      // the row in registers: every load issued before the first is used
      u4 raw[RC][U];
#pragma unroll
      for (int j = 0; j < RC; ++j) load(src, min(lane + 64 * j, nch - 1), raw[j]);
#pragma unroll
      for (int j = 0; j < RC; ++j) {
        if (lane + 64 * j < nch) {
          float x[8];
          widen(raw[j], x);
#pragma unroll
          for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(x[e]));
        }
      }
      mx = wave_max(mx);
      s = mx / 127.0f;
      rs = s > 0.f ? 1.0f / s : 0.f;
#pragma unroll
      for (int j = 0; j < RC; ++j) {
        const int c = lane + 64 * j;
        if (c < nch) {
          float x[8];
          widen(raw[j], x);
          uint32_t lo, hi;
          codes8_i8(x, s, rs, lo, hi, sum);
          dev_store2(dst + 2 * c, lo, hi);
        }
      }
    } else {
      // longer rows: one pass for the maximum, a second (from cache) for the codes
      for (int c = lane; c < nch; c += 64) {
        u4 r[U];
        load(src, c, r);
        float x[8];
        widen(r, x);
#pragma unroll
        for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(x[e]));
      }
      mx = wave_max(mx);
      s = mx / 127.0f;
      rs = s > 0.f ? 1.0f / s : 0.f;
      for (int c = lane; c < nch; c += 64) {
        u4 r[U];
        load(src, c, r);
        float x[8];
        widen(r, x);
        uint32_t lo, hi;
        codes8_i8(x, s, rs, lo, hi, sum);
        dev_store2(dst + 2 * c, lo, hi);
      }
    }
    dev_store(&sa[row], __builtin_bit_cast(uint32_t, s));   // every lane, the same value
    stores_done();                                   // the row is out before it is counted in
    __hip_atomic_fetch_add(&p.sync[SYNC_DONE + row / BM], one, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
  }
}

// The last block to finish resets the counters (every block has passed its
// wait and every wave its row claims by the time it counts itself in).
template <int BM>
__device__ __forceinline__ void fq_finish(const MMParams& p) {
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned total = gridDim.x * gridDim.y;
    if (dev_arrive(&p.sync[SYNC_FIN]) == total - 1) {
      const int mblocks = (p.M + BM - 1) / BM;
      dev_store(&p.sync[SYNC_NEXT], 0u);
      for (int i = 0; i < mblocks; ++i) dev_store(&p.sync[SYNC_DONE + i], 0u);
      dev_store(&p.sync[SYNC_FIN], 0u);
    }
  }
}

template <int KIND, int NTILES, int WM, int OUT, bool BIAS, int FQ>
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
  const int kb = kz * gg.kts;
  const int ke = min(p.KT, kb + gg.kts);
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
    uint8_t* sa = smem + st * S::STAGE;
#pragma unroll
    for (int q = 0; q < S::A_PER_WAVE; ++q) {
      const int ld = wave * S::A_PER_WAVE + q;       // 1 KiB load index within the A tile
      const int row = ld * (64 / RC) + lrow;
      const int c = a_chunk<KIND>(row, lchunk);      // logical chunk for this physical slot
      const int gm = min(m0 + row, p.M - 1);
      const int gk = min(kt * TK + 16 * c, p.K - 16);
      // rows quantized by this launch are read at device scope (sc1), like
      // every other value one block hands to another here
      __builtin_amdgcn_global_load_lds(A + (size_t)gm * p.K + gk, sa + ld * TILE_BYTES, 16, 0,
                                       FQ != 0 ? 16 : 0);
    }
  };
  auto issue_w = [&](int kt, int st) {
    uint8_t* sw = smem + st * S::STAGE + S::A_BYTES;
#pragma unroll
    for (int q = 0; q < S::W_PER_WAVE; ++q) {
      const int tl = q * S::WAVES + wave;            // weight tile within the block
      if (NTILES % S::WAVES != 0 && tl >= NTILES) break;  // wave-uniform
      const int t = min(t0 + tl, p.NT - 1);
      __builtin_amdgcn_global_load_lds(p.Wt + ((size_t)t * p.KT + kt) * TILE_BYTES + lane * 16,
                                       sw + tl * TILE_BYTES, 16, 0, 0);
    }
  };
  auto issue = [&](int kt, int st) {
    issue_a(kt, st);
    issue_w(kt, st);
  };
  auto compute = [&](int st, i4 (&acc)[4][NTW]) {
    const uint8_t* sa = smem + st * S::STAGE;
    const uint8_t* sw = sa + S::A_BYTES;
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

  i4 acc[4][NTW];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int t = 0; t < NTW; ++t) acc[i][t] = i4{0, 0, 0, 0};

  // Two-stage ring: tile i+1 streams into the other stage while tile i is
  // multiplied; the barrier after the wait publishes it to every wave and
  // frees stage i for tile i+2.
  if constexpr (FQ != 0) {
    // the first weight tiles do not depend on the activations: they stream
    // in while the block waits for its m block's quantized rows
    if (nk > 0) issue_w(kb, 0);
    if (wave == 0) {
      if (lane == 0) {
        const unsigned need = (unsigned)min(S::BM, p.M - m0);
        unsigned polls = 0;
        while (dev_count(&p.sync[SYNC_DONE + mb]) < need && ++polls < FQ_SPIN_LIMIT)
          __builtin_amdgcn_s_sleep(8);
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    __syncthreads();
    if (nk > 0) issue_a(kb, 0);
  } else {
    if (nk > 0) issue(kb, 0);
  }
  constexpr bool LP = S::LDS_PARAMS && OUT == W4_OUT_F16;
  float* lws = reinterpret_cast<float*>(smem + S::PARAM_OFF);
  uint16_t* lbias = reinterpret_cast<uint16_t*>(smem + S::PARAM_OFF + NTILES * 16 * 4);
  if constexpr (LP) {
#pragma unroll
    for (int c = tid; c < NTILES * 16; c += S::THREADS) {
      const int n = min(t0 * 16 + c, p.N - 1);
      lws[c] = KIND == KIND_W2A8 ? h2f(p.w_scale16[0]) : p.w_scale[n];
      if constexpr (BIAS) lbias[c] = p.bias[n];
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int i = 0; i < nk; ++i) {
    if (i + 1 < nk) issue(kb + i + 1, (i + 1) & 1);
    compute(i & 1, acc);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }

  // ---- epilogue: lane owns columns n..n+3 of row m for each fragment -------
  const bool vec_ok = (p.N % 4) == 0;
  const int nbase = (t0 + wn * NTW) * 16 + 4 * b;
  float sav[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    sav[i] = OUT == W4_OUT_I32 ? 0.f
             : FQ != 0 ? __builtin_bit_cast(float, dev_load(reinterpret_cast<const uint32_t*>(
                             p.a_scale) + min(m0 + 64 * wm + 16 * i + r, p.M - 1)))
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
  if constexpr (S::SPLIT_OK) {
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
              float o = (float)(acc[i][t][e] >> KindTraits<KIND>::SHIFT) * ws[e] * sav[i];
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
template <int KIND, int NTILES, int WM, int OUT, bool BIAS, int FQ = 0>
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
  if constexpr (FQ != 0) fq_quantize_rows<FQ, 64 * WM>(p);
  gemm_tile<KIND, NTILES, WM, OUT, BIAS, FQ>(p, gg);
  if constexpr (FQ != 0) fq_finish<64 * WM>(p);
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
  if (kind != KIND_W4A8) return GemmCfg{8, 2};       // 2-bit and INT8 weights: 128 x 128
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
  if (kind != KIND_W4A8 && kind != KIND_W2A8 && kind != KIND_W8A8 && kind != KIND_W4A16)
    return false;
  if (M <= 16) return false;
  return gemm_tiles(M, N, gemm_cfg(kind, M, N)) >= 128;
}

inline GemmGrid gemm_grid(int kind, int M, int N, int K, GemmCfg c) {
  const Geometry g = geometry(kind == KIND_W2A8   ? W4_LAYOUT_W2A8
                              : kind == KIND_W8A8 ? W4_LAYOUT_W8A8
                                                  : W4_LAYOUT_W4A8,
                              N, K);
  GemmGrid gg{};
  gg.mblocks = ceil_div(M, 64 * c.wm);
  gg.nblocks = ceil_div(g.NT, c.ntiles);
  gg.tiles = gg.mblocks * gg.nblocks;
  // K is split only for blocks of up to 8 weight tiles, with one arrival
  // counter per tile
  int ks = 1;
  if (c.ntiles <= 8 && gg.tiles <= WS_COUNTER_SLOTS && kind != KIND_W4A16) {
    if (c.ks > 0) ks = c.ks;
    else
      while (gg.tiles * ks < 256 && ceil_div(g.KT, ks * 2) >= 2) ks *= 2;
  }
  gg.kts = ceil_div(g.KT, ks);
  gg.ksplit = ceil_div(g.KT, gg.kts);
  gg.per_xcd = ceil_div(gg.tiles, 8);
  return gg;
}

// counters, then every split's INT32 sums of every block tile
inline size_t gemm_workspace_bytes(int kind, int M, int N, int K, GemmCfg c) {
  const GemmGrid gg = gemm_grid(kind, M, N, K, c);
  if (gg.ksplit == 1) return 0;
  return WS_COUNTERS + (size_t)gg.tiles * gg.ksplit * (64 * c.wm) * (16 * c.ntiles) * sizeof(int32_t);
}

template <int KIND, int NTILES, int WM, int OUT, bool BIAS, int FQ>
int launch_gemm_o(const MMParams& p, const GemmGrid& gg, hipStream_t stream) {
  using S = GemmShape<KIND, NTILES, WM>;
  const dim3 grid(gg.per_xcd * 8, gg.ksplit);
  allow_smem((const void*)&k_gemm<KIND, NTILES, WM, OUT, BIAS, FQ>, S::LDS);
  hipLaunchKernelGGL((k_gemm<KIND, NTILES, WM, OUT, BIAS, FQ>), grid, dim3(S::THREADS), S::LDS,
                     stream, p.Wt, p.A, p.M, p.N, p.K, p.KT, gg.mblocks, gg.nblocks, gg.tiles,
                     gg.per_xcd, gg.kts, p, gg);
  return launch_status();
}

template <int KIND, int NTILES, int WM, int FQ>
int launch_gemm_f(const MMParams& p, const GemmGrid& gg, hipStream_t stream) {
  if constexpr (KIND == KIND_W8A8) {
    if (p.out_dtype == W4_OUT_I8)
      return launch_gemm_o<KIND, NTILES, WM, W4_OUT_I8, false, FQ>(p, gg, stream);
  }
  if (p.out_dtype == W4_OUT_I32)
    return launch_gemm_o<KIND, NTILES, WM, W4_OUT_I32, false, FQ>(p, gg, stream);
  if (p.out_dtype == W4_OUT_F32)
    return launch_gemm_o<KIND, NTILES, WM, W4_OUT_F32, false, FQ>(p, gg, stream);
  if (p.bias) return launch_gemm_o<KIND, NTILES, WM, W4_OUT_F16, true, FQ>(p, gg, stream);
  return launch_gemm_o<KIND, NTILES, WM, W4_OUT_F16, false, FQ>(p, gg, stream);
}

// fq: 0 for int8 activations in p.A; 1 (fp16) or 2 (float32) for rows in
// p.A_in that the kernel quantizes into p.A / p.a_scale first (the caller
// points those at workspace memory and sets p.sync)
template <int KIND, int NTILES, int WM>
int launch_gemm_t(MMParams p, const GemmGrid& gg, void* ws, hipStream_t stream, int fq) {
  p.counters = reinterpret_cast<unsigned*>(ws);
  p.partials = ws ? reinterpret_cast<uint8_t*>(ws) + WS_COUNTERS : nullptr;
  if constexpr (KIND == KIND_W4A8 || KIND == KIND_W2A8) {
    if (fq == 1) return launch_gemm_f<KIND, NTILES, WM, 1>(p, gg, stream);
    if (fq == 2) return launch_gemm_f<KIND, NTILES, WM, 2>(p, gg, stream);
  } else {
    if (fq) return W4_ERR_ARG;
  }
  return launch_gemm_f<KIND, NTILES, WM, 0>(p, gg, stream);
}

// Defined in gemm_launch.hip (a translation unit of its own, so that the
// GEMM instances compile in parallel with the rest of the library).
int launch_gemm_w4a8(const MMParams& p, GemmCfg c, void* ws, hipStream_t stream, int fq);
int launch_gemm_w2a8(const MMParams& p, GemmCfg c, void* ws, hipStream_t stream, int fq);
int launch_gemm_w8a8(const MMParams& p, GemmCfg c, void* ws, hipStream_t stream);
int launch_gemm_w4a16(const MMParams& p, GemmCfg c, hipStream_t stream);  // gemm16.hip

template <int KIND>
int launch_gemm(const MMParams& p, GemmCfg c, void* ws, hipStream_t stream, int fq = 0) {
  if constexpr (KIND == KIND_W4A8) return launch_gemm_w4a8(p, c, ws, stream, fq);
  else if constexpr (KIND == KIND_W2A8) return launch_gemm_w2a8(p, c, ws, stream, fq);
  else if constexpr (KIND == KIND_W8A8) return fq ? W4_ERR_ARG : launch_gemm_w8a8(p, c, ws, stream);
  else if constexpr (KIND == KIND_W4A16) return fq ? W4_ERR_ARG : launch_gemm_w4a16(p, c, stream);
  else return W4_ERR_ARG;
}

}  // namespace w4
