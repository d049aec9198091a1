// Skinny products: more than 16 activation rows but too few output tiles for
// the tiled GEMM (e.g. the ternary M = 128 layers), and every fp16-activation
// product above 16 rows.
//
// Block = 8 waves = one 16-row activation tile x 8 weight n-tiles (128
// output columns). Wave w owns n-tile w of the group over the block's k
// range, so no cross-wave reduction is needed; the block stages its
// activation rows in LDS in k chunks of up to 64 KiB that all 8 waves share,
// which is what the decode kernel (one n-tile per block) cannot do: there
// every n-tile re-reads the same rows. Per chunk: the activation loads and the
// first weight loads are issued together, the rows go to LDS behind one
// barrier, and each wave then streams its weight tiles MAXT at a time through
// registers.
//
// Split K (grid.y = ksplit > 1): block y covers k tiles [y kts, (y+1) kts),
// which gives few-column products enough blocks while every block still
// shares its activation slice across 8 n-tiles. The blocks of a (row tile,
// column group) publish 16 x 128 partial sums at device scope; the last to
// arrive adds them in split order and writes the outputs.
#pragma once

#include "gemv.hpp"

namespace w4 {

constexpr int SKINNY_WAVES = 8;
constexpr int SKINNY_THREADS = SKINNY_WAVES * 64;
constexpr int SKINNY_STAGE = 64 * 1024;            // activation bytes per chunk

// MTB 16-row activation tiles per block (1 to 4): the LDS chunk keeps its
// size at most, so a block of more row tiles stages a shorter k range per
// chunk: the largest power of two of k tiles that fits (a split block pads
// each row's piece count to a power of two, so a row's pieces must be one).
template <int KIND, int MTB = 1>
__host__ __device__ constexpr int skinny_chunk_tiles() {
  int ct = 1;
  while (2 * ct * 16 * MTB * AStage<KIND>::TILE_ROWB <= SKINNY_STAGE) ct *= 2;
  return ct;
}

template <int KIND, int MTB = 1>
constexpr size_t skinny_smem() {
  return (size_t)16 * MTB * (skinny_chunk_tiles<KIND, MTB>() * AStage<KIND>::TILE_ROWB + 16);
}

// SPLIT selects the k-split instance; without it the kernel covers the whole K
// with the staging and epilogue of the unsplit kernel exactly. MTB > 1 makes
// each block cover MTB 16-row activation tiles: every weight tile a wave
// loads and unpacks then feeds MTB MFMA chains, which divides the weight
// traffic and the block count of many-row products by MTB (the ternary
// M = 128 layers at N = 8640 need 544 one-tile blocks, 272 two-tile blocks,
// or 204 three-tile blocks, the only count of these within one block per CU).
//
// The fields the first loads depend on come as leading scalar arguments,
// preloaded into SGPRs (see k_gemv); per_xcd is the grid size / 8, and the
// k-tile counts follow from K and the kind's tile extent.
template <int KIND, int MAXT, bool SPLIT = false, int MTB = 1>
__global__ __launch_bounds__(SKINNY_THREADS) void k_skinny(const uint8_t* Wt, const void* A,
                                                           const uint16_t* St, const uint8_t* Zt,
                                                           int M, int K, int NT, int kts,
                                                           int ngroups, int per_xcd,
                                                           const MMParams pin) {
  using AS = AStage<KIND>;
  constexpr bool A16 = KIND == KIND_W4A16 || KIND == KIND_W2A16;
  constexpr bool GRP = KIND == KIND_W4A16;
  constexpr int AC = KindTraits<KIND>::A_CHUNKS;
  constexpr int RB = 16 * MTB;                       // activation rows per block
  constexpr int CT = skinny_chunk_tiles<KIND, MTB>();  // k tiles per staged chunk
  constexpr int ROWB = CT * AS::TILE_ROWB;           // staged bytes per row
  constexpr int SSTRIDE = ROWB + 16;                 // padded: conflict-free fragment reads
  constexpr int APER = RB * ROWB / 16 / SKINNY_THREADS;  // 16-byte staging loads per thread
  static_assert(RB * ROWB % (16 * SKINNY_THREADS) == 0, "staging chunk");
  static_assert(MTB >= 1 && MTB <= 4, "row tiles per block");
  typedef typename std::conditional<float_acc<KIND>(), f4, i4>::type Acc;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  MMParams p = pin;
  p.Wt = Wt;
  p.A = A;
  p.St = St;
  p.Zt = Zt;
  p.M = M;
  p.K = K;
  p.NT = NT;
  p.kts = kts;
  p.KT = (K + KindTraits<KIND>::TILE_K - 1) / KindTraits<KIND>::TILE_K;
  p.KQ = (p.KT + 3) / 4;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, b = lane >> 4;
  // block id -> (n group, m block): consecutive ids of one XCD walk the m
  // blocks of one n group, so the group's weight tiles stay in that XCD's L2
  const int mtiles = (p.M + RB - 1) / RB;            // blocks of RB rows
  const int id = blockIdx.x, xcd = id & 7, local = id >> 3;
  const int seq = xcd * per_xcd + local;             // the grid is 8 * per_xcd blocks
  const int grp = small_div(seq, mtiles), mtile = seq - grp * mtiles;
  if (local >= per_xcd || grp >= ngroups) return;    // block-uniform
  const int tile = grp * SKINNY_WAVES + wave;        // this wave's n tile
  const bool live_tile = tile < p.NT;                // wave-uniform
  const int rows = min(RB, p.M - mtile * RB);
  const uint8_t* Ab = reinterpret_cast<const uint8_t*>(p.A);
  const size_t arow_bytes = (size_t)p.K * AS::ESZ;
  const int cpr = ROWB / 16;                         // 16-byte chunks per staged row
  const int kb = SPLIT ? blockIdx.y * p.kts : 0;     // this block's k tiles [kb, ke)
  const int ke = SPLIT ? min(p.KT, kb + p.kts) : p.KT;

  Acc acc[MTB];
#pragma unroll
  for (int j = 0; j < MTB; ++j) acc[j] = Acc{};
  // ---- activation loads of the chunk at kc (rows past M clamp, k past K
  // zero): 16-byte pieces in row-major order, each row padded to a
  // power-of-two piece count lg2 >= the ct tiles the chunk holds (a full chunk
  // has no padding; a short k range per block under a k split would otherwise
  // load and store a full chunk for a fraction of it). Padding slots re-read
  // piece 0, so that the loads stay unconditional and the wait counts exact.
  // (the unsplit kernel deals the full chunk's pieces, zeroing those past
  // the chunk's tiles). A chunk at kc >= ke (the prefetch after the last one)
  // reads the first 16 bytes of A in every slot: always in range, one cache
  // line, and the count of loads in flight stays the same on every path.
  auto chunk_geo = [&](int kc, int& ct, int& cw, int& lg) {
    ct = min(CT, ke - kc);                           // k tiles in this chunk
    cw = ct * (AS::TILE_ROWB / 16);                  // pieces per row in use
    lg = cw > 1 ? 32 - __builtin_clz((unsigned)(cw - 1)) : 0;
  };
  u4 stage[APER];
  auto load_chunk = [&](int kc) {
    const bool live = kc < ke;                       // block-uniform
    int ct, cw, lg;
    chunk_geo(live ? kc : kb, ct, cw, lg);
    const int need = RB << lg;
    const size_t kbyte0 = (size_t)kc * AS::TILE_ROWB;
#pragma unroll
    for (int i = 0; i < APER; ++i) {
      const int c = tid + i * SKINNY_THREADS;
      int row, col;
      if constexpr (SPLIT) {
        const bool u = c < need && (c & ((1 << lg) - 1)) < cw;
        const int cc = u ? c : 0;
        row = cc >> lg;
        col = cc & ((1 << lg) - 1);
      } else {
        row = c / cpr;
        col = c - row * cpr;
      }
      // past K (or past the chunk's tiles): clamp into the row, zeroed below
      const size_t off = min(kbyte0 + (size_t)col * 16, arow_bytes - 16);
      const int gm = min(mtile * RB + row, p.M - 1);
      const size_t at = live ? (size_t)gm * arow_bytes + off : 0;
      stage[i] = *reinterpret_cast<const u4*>(Ab + at);
    }
  };
  // Blocks of three or four row tiles (one per CU, several chunks per block)
  // load each next chunk while the current one is multiplied; smaller blocks
  // run two per CU, where the registers that prefetch holds would cost
  // occupancy (M=128 N=8640 K=3200 on MI355X: W2A8 at three tiles 13.5 ->
  // 12.9 us with it, W2A16 20.6 -> 19.6; at one tile W2A8 13.8 -> 17.7 us).
  constexpr bool PF = MTB >= 3;
  if constexpr (PF) load_chunk(kb);
  for (int kc = kb; kc < ke; kc += CT) {
    if constexpr (!PF) load_chunk(kc);
    int ct, cw, lg;
    chunk_geo(kc, ct, cw, lg);
    const size_t kbyte0 = (size_t)kc * AS::TILE_ROWB;
    const int need = RB << lg;
    auto used = [&](int c) { return c < need && (c & ((1 << lg) - 1)) < cw; };
    for (int pass = 0; pass * MAXT < ct; ++pass) {
      const int pn = min(MAXT, ct - pass * MAXT);    // tiles in this pass (uniform)
      // ---- this wave's weight tiles (unconditional: dead slots re-read tile 0)
      u4 wv[MAXT];
      uint16_t sv[MAXT];
      uint8_t zv[MAXT];
#pragma unroll
      for (int u = 0; u < MAXT; ++u) {
        const bool live = live_tile && u < pn;
        const int kt = kc + pass * MAXT + u;
        const size_t ti = live ? (size_t)tile * p.KT + kt : 0;
        wv[u] = *reinterpret_cast<const u4*>(p.Wt + ti * TILE_BYTES + lane * 16);
        if constexpr (GRP) {
          const size_t mi =
              live ? (((size_t)tile * p.KQ + (kt >> 2)) * TILE_N + r) * 4 + (kt & 3) : 0;
          sv[u] = p.St[mi];
          zv[u] = p.Zt[mi];
        } else {
          sv[u] = 0;
          zv[u] = 0;
        }
      }
      if (pass == 0) {
        // ---- rows to LDS: wait for the previous chunk's readers first ----
        __syncthreads();
#pragma unroll
        for (int i = 0; i < APER; ++i) {
          const int c = tid + i * SKINNY_THREADS;
          if constexpr (SPLIT) {
            if (used(c)) {
              const int row = c >> lg, col = c & ((1 << lg) - 1);
              u4 v = stage[i];
              if (kbyte0 + (size_t)col * 16 >= arow_bytes) v = u4{0u, 0u, 0u, 0u};
              *reinterpret_cast<u4*>(smem + row * SSTRIDE + col * 16) = v;
            }
          } else {
            const int row = c / cpr, col = c - row * cpr;
            u4 v = stage[i];
            if (kbyte0 + (size_t)col * 16 >= arow_bytes || col * 16 >= ct * AS::TILE_ROWB)
              v = u4{0u, 0u, 0u, 0u};
            *reinterpret_cast<u4*>(smem + row * SSTRIDE + col * 16) = v;
          }
        }
        // (prefetch) the next chunk's rows stream in while this one is multiplied (its
        // loads are issued after this pass's weight loads, so the matrix
        // cores of this pass do not wait for them)
        if constexpr (PF) load_chunk(kc + CT);
        __syncthreads();
      }
      if (!live_tile) continue;                      // wave-uniform: nothing to multiply
#pragma unroll
      for (int u = 0; u < MAXT; ++u) {
        if (u >= pn) continue;                       // uniform
        const int kl = pass * MAXT + u;              // tile index within the chunk
#pragma unroll
        for (int t = 0; t < MTB; ++t) {
          const u4* src = reinterpret_cast<const u4*>(smem + (16 * t + r) * SSTRIDE +
                                                      kl * AS::TILE_ROWB + (AS::TILE_ROWB / 4) * b);
          u4 af[AC];
#pragma unroll
          for (int j = 0; j < AC; ++j) af[j] = src[j];
          tile_mma<KIND>(wv[u], af, sv[u], zv[u], acc[t]);
        }
      }
    }
  }

  // ---- epilogue: lane holds output column (lane & 15), rows 4*(lane >> 4)+e
  const int n = tile * 16 + r;
  if constexpr (!SPLIT) {
    if (!live_tile || n >= p.N) return;
#pragma unroll
    for (int t = 0; t < MTB; ++t) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 16 * t + 4 * b + e;
        if (row >= rows) continue;
        const int m = mtile * RB + row;
        const auto v = acc[t][e];                    // scalar copy before any bit cast
        if constexpr (A16) {
          store_out<KIND>(p, m, n, v, 0, 0.f);
        } else if constexpr (float_acc<KIND>()) {
          store_out<KIND>(p, m, n, v, 0, p.a_scale[m]);
        } else {
          store_out<KIND>(p, m, n, 0.f, v, p.a_scale[m]);
        }
      }
    }
    return;
  }
  auto store = [&](int row, float fv, int iv) {
    const int m = mtile * RB + row;
    if constexpr (A16) store_out<KIND>(p, m, n, fv, 0, 0.f);
    else store_out<KIND>(p, m, n, fv, iv, p.a_scale[m]);
  };

  // ---- split K: publish this block's RB x 128 partial sums (every wave, so
  // that all of them reach the barriers), the last block adds them up. The
  // blocks of a (row tile, column group) hold the same outputs in the same
  // registers, so the sums are kept in register order: word pair q of thread
  // tid of split z at ((slot * ksplit + z) * Q2 + q) * THREADS + tid, and a
  // wave instruction moves 512 contiguous bytes.
  constexpr int Q2 = 2 * MTB;                        // 64-bit words per thread
  const size_t slot = (size_t)mtile * ngroups + grp;
  uint64_t* slot_part = reinterpret_cast<uint64_t*>(p.partials) +
                        slot * p.ksplit * Q2 * SKINNY_THREADS;
  auto word = [&](int z, int q) {
    return reinterpret_cast<uint32_t*>(slot_part + ((size_t)z * Q2 + q) * SKINNY_THREADS + tid);
  };
#pragma unroll
  for (int t = 0; t < MTB; ++t) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const auto lo = acc[t][2 * h], hi = acc[t][2 * h + 1];
      dev_store2(word(blockIdx.y, 2 * t + h), __builtin_bit_cast(uint32_t, lo),
                 __builtin_bit_cast(uint32_t, hi));
    }
  }
  __shared__ int last;
  stores_done();
  __syncthreads();
  if (tid == 0) last = dev_arrive(&p.counters[slot]) == (unsigned)(p.ksplit - 1);
  __syncthreads();
  if (!last) return;
  if (tid == 0) dev_store(&p.counters[slot], 0u);   // every split has counted in
  if (!live_tile || n >= p.N) return;
  // Sum every split's value in split order (float sums then do not depend on
  // which block finishes), 8 splits per batch: every load of a batch is issued
  // before any is added, so a batch costs one round trip to the level all
  // XCDs share.
  float fs[MTB][4] = {};
  int is[MTB][4] = {};
  for (int z0 = 0; z0 < p.ksplit; z0 += 8) {
    // keeps the compiler from hoisting the next batch's loads (and their
    // registers) above this batch's additions
    asm volatile("" ::: "memory");
    uint64_t v[8][Q2];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int q = 0; q < Q2; ++q) v[j][q] = dev_load2(word(min(z0 + j, p.ksplit - 1), q));
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (z0 + j >= p.ksplit) break;
#pragma unroll
      for (int t = 0; t < MTB; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t bits = (uint32_t)(v[j][2 * t + e / 2] >> (32 * (e & 1)));
          if constexpr (float_acc<KIND>()) fs[t][e] += __builtin_bit_cast(float, bits);
          else is[t][e] += (int)bits;
        }
    }
  }
#pragma unroll
  for (int t = 0; t < MTB; ++t) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 16 * t + 4 * b + e;
      if (row < rows) store(row, fs[t][e], is[t][e]);
    }
  }
}

}  // namespace w4
