// Prefill-side kernel for fp16 activations and group-quantized 4-bit weights
// (W4A16, M > 16): C[M,N] = A[M,K] x W[N,K]^T on the CDNA4 fp16 matrix cores.
//
// Dataflow (BitBLAS page, data-type table row FP16 x INT4 and "Advanced
// features 2" (group scales and zeros); INT4 page, Part 1 step 3): for each
// 128-k tile (one quantization group), a block copies its fp16 activation tile
// (BM x 128 halves) and its prepacked weight tiles (still 4-bit, 1 KiB per 16
// columns) from global memory into one of two LDS stages while the matrix
// cores work on the other. Each wave widens a weight fragment to fp16
// (q - z) in registers (the 0x6400 exponent trick, exact), multiplies it with
// its activation fragments on v_mfma_f32_16x16x32_f16 (exact fp16 products,
// float32 sums), and scales each group's partial sum by the group's fp16
// scale in float32 before adding it to the accumulator, the order the decode
// kernel uses. Epilogue: + bias, fp16 store.
//
// Block: 2*WN waves as 2 (m) x WN (n), block tile 128 rows x 16*NTILES
// columns, wave tile 64 x 16*NTILES/WN; one block per CU (the two stages take
// 2 x 48 KiB of LDS at NTILES = 16, 2 x 54 KiB at 22). Eight waves (WN = 4)
// give each SIMD two, so that one wave's unpacking and LDS reads overlap the
// other's matrix-core work. Activations are the MFMA row operand and weights the
// column operand, so a lane's accumulators all belong to one output column n
// (the weight row it unpacks), whose scale and zero it loads itself.
// Blocks are dealt to the XCDs as in the INT8 GEMM.

#include "gemm.hpp"

namespace w4 {

template <int NTILES, int WN>
struct Gemm16Shape {
  static constexpr int WAVES = 2 * WN;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int BM = 128;
  static constexpr int TK = 128;                           // k per stage = one group
  static constexpr int ROWB = TK * 2;                      // staged bytes per activation row
  static constexpr int A_BYTES = BM * ROWB;                // 32 KiB, XOR-swizzled 16-byte chunks
  static constexpr int A_LOADS = A_BYTES / TILE_BYTES;     // 32 wave loads of 1 KiB
  static constexpr int A_PER_WAVE = A_LOADS / WAVES;
  static constexpr int W_BYTES = NTILES * TILE_BYTES;
  static constexpr int W_PER_WAVE = (NTILES + WAVES - 1) / WAVES;
  static_assert(NTILES % WN == 0, "the n waves split the block's columns");
  static_assert(A_LOADS % WAVES == 0, "activation loads per wave");
  static constexpr int NTW = NTILES / WN;                  // column fragments per wave
  // the group scales and zeros of the stage's 128-k group: one 4-byte word
  // per (tile, row) for each, copied straight to LDS like the tiles; a word
  // holds the scales of groups 2h, 2h+1 (h = group / 2 within its quad) or the
  // zeros of the quad's four groups
  static constexpr int META_ITEMS = 2 * NTILES * TILE_N;
  static constexpr int META_PER_WAVE = (META_ITEMS + 64 * WAVES - 1) / (64 * WAVES);
  static constexpr int META_BYTES = META_PER_WAVE * WAVES * 256;
  static constexpr int STAGE = A_BYTES + W_BYTES + META_BYTES;
  // three stages where they fit and every wave issues the same loads per
  // tile (so that a fixed wait count covers exactly one tile's loads)
  static constexpr int LOADS = A_PER_WAVE + W_PER_WAVE + META_PER_WAVE;  // per wave per tile
  static constexpr int STAGES = (3 * STAGE <= 160 * 1024 && NTILES % WAVES == 0) ? 3 : 2;
  // fp16 epilogue staging: per wave and pass, 32 rows x 16*NTW columns
  static constexpr int EPI_ROW = NTW * 32 + 16;            // padded row bytes
  static constexpr int EPI = WAVES * 32 * EPI_ROW;
  static constexpr int LDS = STAGES * STAGE > EPI ? STAGES * STAGE : EPI;
  static_assert(LDS <= 160 * 1024, "LDS exceeds the CU");
};

// physical 16-byte chunk of logical chunk c in staged activation row `row`:
// 256-byte rows all start on bank 0, so the 16 rows of a fragment read are
// spread by the row index
__device__ __forceinline__ int a16_chunk(int row, int c) { return c ^ (row & 15); }

// The block's work (a device function: the kernel below only forwards its
// arguments, so that its host-side stub holds no device assembly).
template <int NTILES, int WN, bool BIAS>
__device__ __forceinline__ void gemm16_tile(const uint8_t* Wt, const uint16_t* St,
                                            const uint8_t* Zt, const void* Av, int M, int N,
                                            int K, int mblocks, int nblocks, int per_xcd,
                                            const MMParams& pin) {
  using S = Gemm16Shape<NTILES, WN>;
  constexpr int NTW = S::NTW;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int KT = K / S::TK, KQ = (KT + 3) / 4, NT = (N + TILE_N - 1) / TILE_N;

  // ---- block -> (m block, n block), as k_gemm deals them ------------------
  const int id = blockIdx.x;
  const int xcd = id & 7, local = id >> 3;
  const int tix = xcd * per_xcd + local;
  if (local >= per_xcd || tix >= mblocks * nblocks) return;
  int nb, mb;
  if (mblocks % 2 == 0) {
    const int mh = mblocks / 2;
    const int half = small_div(tix, nblocks * mh);
    const int rem = tix - half * nblocks * mh;
    nb = small_div(rem, mh);
    mb = half * mh + (rem - nb * mh);
  } else {
    nb = small_div(tix, mblocks);
    mb = tix - nb * mblocks;
  }

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;            // wn in [0, WN)
  const int r = lane & 15, b = lane >> 4;
  const int m0 = mb * S::BM;
  const int t0 = nb * NTILES;
  const uint8_t* A = reinterpret_cast<const uint8_t*>(Av);
  const size_t arow = (size_t)K * 2;

  // ---- direct global -> LDS copies of k tile kt into stage st -------------
  // A load: 1 KiB = 4 rows x 16 chunks (lane l: row l / 16, physical chunk
  // l % 16, holding logical chunk a16_chunk(row, l % 16)); rows past M read the
  // last row (never stored). W load: one 1 KiB tile (columns past N are zero
  // codes from the prepack, never stored).
  auto issue = [&](int kt, int st) {
    uint8_t* sa = smem + st * S::STAGE;
#pragma unroll
    for (int q = 0; q < S::A_PER_WAVE; ++q) {
      const int ld = wave * S::A_PER_WAVE + q;
      const int row = ld * 4 + (lane >> 4);
      const int c = a16_chunk(row, lane & 15);
      const int gm = min(m0 + row, M - 1);
      __builtin_amdgcn_global_load_lds(A + (size_t)gm * arow + (size_t)kt * S::ROWB + 16 * c,
                                       sa + ld * TILE_BYTES, 16, 0, 0);
    }
    uint8_t* sw = sa + S::A_BYTES;
#pragma unroll
    for (int q = 0; q < S::W_PER_WAVE; ++q) {
      const int tl = q * S::WAVES + wave;
      if (NTILES % S::WAVES != 0 && tl >= NTILES) break;      // wave-uniform
      const int t = min(t0 + tl, NT - 1);
      __builtin_amdgcn_global_load_lds(Wt + ((size_t)t * KT + kt) * TILE_BYTES + lane * 16,
                                       sw + tl * TILE_BYTES, 16, 0, 0);
    }
    // scales: item (tile tl, row rr) -> the word with groups 2h, 2h+1;
    // zeros: item NTILES*16 + (tl, rr) -> the word with the quad's zeros
    // (items past the end re-read the last one, for equal load counts)
    uint8_t* sm = sw + S::W_BYTES;
#pragma unroll
    for (int q = 0; q < S::META_PER_WAVE; ++q) {
      const int item = min((q * S::WAVES + wave) * 64 + lane, S::META_ITEMS - 1);
      const int zpart = item >= NTILES * TILE_N;
      const int it = item - zpart * NTILES * TILE_N;
      const int t = min(t0 + it / TILE_N, NT - 1), rr = it % TILE_N;
      const size_t rec = ((size_t)t * KQ + (kt >> 2)) * TILE_N + rr;
      const uint8_t* src = zpart ? Zt + rec * 4
                                 : reinterpret_cast<const uint8_t*>(St) + rec * 8 + (kt & 2) * 2;
      __builtin_amdgcn_global_load_lds(src, sm + (q * S::WAVES + wave) * 256, 4, 0, 0);
    }
  };

  f4 acc[4][NTW];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int t = 0; t < NTW; ++t) acc[i][t] = f4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int st, int kt) {
    const uint8_t* sa = smem + st * S::STAGE;
    const uint8_t* sw = sa + S::A_BYTES + (wn * NTW) * TILE_BYTES + lane * 16;
    // this lane's column (row r of each of its weight tiles): scale and zero
    const uint8_t* sm = sa + S::A_BYTES + S::W_BYTES;
    uint16_t sv[NTW];
    uint8_t zv[NTW];
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      const int it = (wn * NTW + t) * TILE_N + r;
      sv[t] = *reinterpret_cast<const uint16_t*>(sm + it * 4 + (kt & 1) * 2);
      zv[t] = sm[(NTILES * TILE_N + it) * 4 + (kt & 3)];
    }
    // activation fragments: row frag i, k step j -> lane (r, b) holds row
    // 64 wm + 16 i + r, k = 32 b + 8 j .. + 7 (the k order of the weight words)
    h8 af[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 64 * wm + 16 * i + r;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        af[i][j] = *reinterpret_cast<const h8*>(sa + row * S::ROWB + 16 * a16_chunk(row, 4 * b + j));
    }
    u4 wn_next = *reinterpret_cast<const u4*>(sw);
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      // least progress first (as in k_gemm): the two waves of a SIMD run the
      // same fragment sequence, and a wave lowers its priority as it gets
      // through its fragments, so the one that is behind is issued first
      if (t == 0 || (4 * t) / NTW != (4 * (t - 1)) / NTW) {
        switch ((4 * t) / NTW) {
          case 0: __builtin_amdgcn_s_setprio(3); break;
          case 1: __builtin_amdgcn_s_setprio(2); break;
          case 2: __builtin_amdgcn_s_setprio(1); break;
          default: __builtin_amdgcn_s_setprio(0); break;
        }
      }
      const u4 w = wn_next;
      if (t + 1 < NTW) wn_next = *reinterpret_cast<const u4*>(sw + (t + 1) * TILE_BYTES);
      const _Float16 z = (_Float16)(float)zv[t];
      const _Float16 zl = -((_Float16)1024.0f + z);
      const _Float16 zh = -((_Float16)64.0f + z);
      const h2 zlo = {zl, zl}, zhi = {zh, zh};
      h8 bf[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t wj = w[j];
        bf[j] = unpack_w4_f16(wj, zlo, zhi);
      }
      f4 part[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) part[i] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          part[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i][j], bf[j], part[i], 0, 0, 0);
      const float s = h2f(sv[t]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[i][t][e] = fmaf(part[i][e], s, acc[i][t][e]);
    }
  };

  // Ring of S::STAGES stages: tile i + STAGES - 1 streams into a free stage
  // (and its group scales and zeros into registers) while tile i is
  // multiplied; at the end of step i the wave waits for tile i + 1's loads
  // only (the later tiles' stay in flight), and the barrier publishes them
  // and frees stage i.
  constexpr int ST = S::STAGES;
#pragma unroll
  for (int q = 0; q < ST - 1; ++q)
    if (q < KT) issue(q, q);
  auto wait_next = [&](bool later_in_flight) {
    // vmcnt counts this wave's loads: LOADS per tile, all of the later
    // tiles' may still be outstanding
    if (ST == 3 && later_in_flight) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(S::LOADS) : "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  };
  // The barrier is written out: __syncthreads() would also wait for every
  // outstanding load (its release fence), which would drain the tiles that
  // are meant to stay in flight. Each wave has waited for its own share of
  // tile i + 1 (the LDS-direct loads count as done once written to LDS) and
  // for its LDS reads; the memory clobber keeps the compiler from moving LDS
  // accesses across.
  auto barrier = [] { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };
  wait_next(ST == 3 && KT > 1);
  barrier();
  int cur = 0;                                      // the stage of tile kt
  for (int kt = 0; kt < KT; ++kt) {
    if (kt + ST - 1 < KT) issue(kt + ST - 1, cur == 0 ? ST - 1 : cur - 1);
    compute(cur, kt);
    wait_next(kt + ST - 1 < KT);
    barrier();
    cur = cur + 1 == ST ? 0 : cur + 1;
  }

  // ---- epilogue: lane holds rows 64 wm + 16 i + 4 b + e of column n -------
  const MMParams& p = pin;
  uint16_t* C = reinterpret_cast<uint16_t*>(p.C);
  const int nw = (t0 + wn * NTW) * 16;                      // first column of the wave tile
  float bcol[NTW];
#pragma unroll
  for (int t = 0; t < NTW; ++t) bcol[t] = BIAS ? h2f(p.bias[min(nw + 16 * t + r, N - 1)]) : 0.f;
  if ((N % 8) == 0) {
    // stage 32 rows x 16*NTW columns per pass, then store 16-byte row chunks
    constexpr int WC = NTW * 16;
    uint8_t* cw = smem + wave * 32 * S::EPI_ROW;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int ii = 0; ii < 2; ++ii) {
        const int i = 2 * h + ii;
#pragma unroll
        for (int t = 0; t < NTW; ++t)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float v = acc[i][t][e] + bcol[t];
            *reinterpret_cast<uint16_t*>(cw + (16 * ii + 4 * b + e) * S::EPI_ROW +
                                         (16 * t + r) * 2) = f2h(v);
          }
      }
#pragma unroll
      for (int q = 0; q < 32 * WC / 8 / 64; ++q) {
        const int c = q * 64 + lane;
        const int row = c / (WC / 8), c8 = c % (WC / 8);
        const u4 v = *reinterpret_cast<const u4*>(cw + row * S::EPI_ROW + c8 * 16);
        const int m = m0 + 64 * wm + 32 * h + row, n = nw + 8 * c8;
        if (m < M && n < N) *reinterpret_cast<u4*>(C + (size_t)m * N + n) = v;
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int t = 0; t < NTW; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = m0 + 64 * wm + 16 * i + 4 * b + e, n = nw + 16 * t + r;
        if (m < M && n < N) C[(size_t)m * N + n] = f2h(acc[i][t][e] + bcol[t]);
      }
}

// The fields the block's first loads depend on come as leading scalar
// arguments, preloaded into SGPRs (see k_gemv); KT and KQ follow from K.
template <int NTILES, int WN, bool BIAS>
__global__ __launch_bounds__(128 * WN, 1) void k_gemm16(const uint8_t* Wt, const uint16_t* St,
                                                        const uint8_t* Zt, const void* Av, int M,
                                                        int N, int K, int mblocks, int nblocks,
                                                        int per_xcd, const MMParams pin) {
  gemm16_tile<NTILES, WN, BIAS>(Wt, St, Zt, Av, M, N, K, mblocks, nblocks, per_xcd, pin);
}

template <int NTILES, int WN, bool BIAS>
int launch_gemm16_o(const MMParams& p, const GemmGrid& gg, hipStream_t stream) {
  using S = Gemm16Shape<NTILES, WN>;
  allow_smem((const void*)&k_gemm16<NTILES, WN, BIAS>, S::LDS);
  hipLaunchKernelGGL((k_gemm16<NTILES, WN, BIAS>), dim3(gg.per_xcd * 8), dim3(S::THREADS),
                     S::LDS, stream, p.Wt, p.St, p.Zt, p.A, p.M, p.N, p.K, gg.mblocks,
                     gg.nblocks, gg.per_xcd, p);
  return launch_status();
}

template <int NTILES, int WN>
int launch_gemm16_b(const MMParams& p, const GemmGrid& gg, hipStream_t stream) {
  return p.bias ? launch_gemm16_o<NTILES, WN, true>(p, gg, stream)
                : launch_gemm16_o<NTILES, WN, false>(p, gg, stream);
}

// Block shapes by GemmCfg.ntiles (128 rows each, GemmCfg.wm = 2): 128 x 256
// and 128 x 384 on eight waves, 128 x 352 on four (22 tiles do not split
// four ways).
int launch_gemm_w4a16(const MMParams& p, GemmCfg c, hipStream_t stream) {
  const GemmGrid gg = gemm_grid(KIND_W4A16, p.M, p.N, p.K, c);
  if (gg.ksplit != 1 || (p.K % 128) != 0 || c.wm != 2) return W4_ERR_ARG;
  if (c.ntiles == 22) return launch_gemm16_b<22, 2>(p, gg, stream);
  if (c.ntiles == 24) return launch_gemm16_b<24, 4>(p, gg, stream);
  if (c.ntiles == 16) return launch_gemm16_b<16, 4>(p, gg, stream);
  return W4_ERR_ARG;
}

}  // namespace w4
