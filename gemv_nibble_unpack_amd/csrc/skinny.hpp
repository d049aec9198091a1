// Skinny products: more than 16 activation rows but too few output tiles for
// the tiled GEMM (e.g. the ternary M = 128 layers), and every fp16-activation
// product above 16 rows.
//
// Block = 8 waves = one 16-row activation tile x 8 weight n-tiles (128
// output columns). Wave w owns n-tile w of the group over the whole K, so no
// cross-wave reduction is needed; the block stages its activation rows in LDS
// in k chunks of up to 64 KiB that all 8 waves share, which is what the
// decode kernel (one n-tile per block) cannot do: there every n-tile re-reads
// the same rows. Per chunk: the activation loads and the first weight loads
// are issued together, the rows go to LDS behind one barrier, and each wave
// then streams its weight tiles MAXT at a time through registers.
#pragma once

#include "gemv.hpp"

namespace w4 {

constexpr int SKINNY_WAVES = 8;
constexpr int SKINNY_THREADS = SKINNY_WAVES * 64;
constexpr int SKINNY_STAGE = 64 * 1024;            // activation bytes per chunk

template <int KIND>
__host__ __device__ constexpr int skinny_chunk_tiles() {
  return SKINNY_STAGE / (16 * AStage<KIND>::TILE_ROWB);
}

template <int KIND>
constexpr size_t skinny_smem() {
  return (size_t)16 * (skinny_chunk_tiles<KIND>() * AStage<KIND>::TILE_ROWB + 16);
}

template <int KIND, int MAXT>
__global__ __launch_bounds__(SKINNY_THREADS) void k_skinny(const MMParams p, int ngroups) {
  using AS = AStage<KIND>;
  constexpr bool A16 = KIND == KIND_W4A16 || KIND == KIND_W2A16;
  constexpr bool GRP = KIND == KIND_W4A16;
  constexpr int AC = KindTraits<KIND>::A_CHUNKS;
  constexpr int CT = skinny_chunk_tiles<KIND>();     // k tiles per staged chunk
  constexpr int ROWB = CT * AS::TILE_ROWB;           // staged bytes per row
  constexpr int SSTRIDE = ROWB + 16;                 // padded: conflict-free fragment reads
  constexpr int APER = 16 * ROWB / 16 / SKINNY_THREADS;  // 16-byte staging loads per thread
  static_assert(16 * ROWB % (16 * SKINNY_THREADS) == 0, "staging chunk");
  typedef typename std::conditional<float_acc<KIND>(), f4, i4>::type Acc;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  fetch_args(p);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, b = lane >> 4;
  // block id -> (n group, m tile): consecutive ids of one XCD walk the m tiles
  // of one n group, so the group's weight tiles stay in that XCD's L2
  const int mtiles = (p.M + 15) / 16;
  const int id = blockIdx.x, xcd = id & 7, local = id >> 3;
  const int per_xcd = (int)(gridDim.x >> 3);         // grid is a multiple of 8
  const int seq = xcd * per_xcd + local;
  const int grp = seq / mtiles, mtile = seq - grp * mtiles;
  if (local >= per_xcd || grp >= ngroups) return;    // block-uniform
  const int tile = grp * SKINNY_WAVES + wave;        // this wave's n tile
  const bool live_tile = tile < p.NT;                // wave-uniform
  const int rows = min(16, p.M - mtile * 16);
  const uint8_t* Ab = reinterpret_cast<const uint8_t*>(p.A);
  const size_t arow_bytes = (size_t)p.K * AS::ESZ;
  const int cpr = ROWB / 16;                         // 16-byte chunks per staged row

  Acc acc = Acc{};
  for (int kc = 0; kc < p.KT; kc += CT) {
    const int ct = min(CT, p.KT - kc);               // k tiles in this chunk
    const size_t kbyte0 = (size_t)kc * AS::TILE_ROWB;
    // ---- activation loads of the chunk (rows past M clamp, k past K zero) --
    u4 stage[APER];
#pragma unroll
    for (int i = 0; i < APER; ++i) {
      const int c = tid + i * SKINNY_THREADS;
      const int row = c / cpr, col = c - row * cpr;
      // past K (or past the chunk's last tile): clamp into the row, zeroed below
      const size_t off = min(kbyte0 + (size_t)col * 16, arow_bytes - 16);
      const int gm = min(mtile * 16 + row, p.M - 1);
      stage[i] = *reinterpret_cast<const u4*>(Ab + (size_t)gm * arow_bytes + off);
    }
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
          const int row = c / cpr, col = c - row * cpr;
          u4 v = stage[i];
          if (kbyte0 + (size_t)col * 16 >= arow_bytes || col * 16 >= ct * AS::TILE_ROWB)
            v = u4{0u, 0u, 0u, 0u};
          *reinterpret_cast<u4*>(smem + row * SSTRIDE + col * 16) = v;
        }
        __syncthreads();
      }
      if (!live_tile) continue;                      // wave-uniform: nothing to multiply
      const uint8_t* arow = smem + r * SSTRIDE;
#pragma unroll
      for (int u = 0; u < MAXT; ++u) {
        if (u >= pn) continue;                       // uniform
        const int kl = pass * MAXT + u;              // tile index within the chunk
        const u4* src = reinterpret_cast<const u4*>(arow + kl * AS::TILE_ROWB +
                                                    (AS::TILE_ROWB / 4) * b);
        u4 af[AC];
#pragma unroll
        for (int j = 0; j < AC; ++j) af[j] = src[j];
        tile_mma<KIND>(wv[u], af, sv[u], zv[u], acc);
      }
    }
  }

  // ---- epilogue: lane holds output column (lane & 15), rows 4*(lane >> 4)+e
  if (!live_tile) return;
  const int n = tile * 16 + r;
  if (n >= p.N) return;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int row = 4 * b + e;
    if (row >= rows) continue;
    const int m = mtile * 16 + row;
    const auto v = acc[e];                           // scalar copy before any bit cast
    if constexpr (A16) {
      store_out<KIND>(p, m, n, v, 0, 0.f);
    } else if constexpr (float_acc<KIND>()) {
      store_out<KIND>(p, m, n, v, 0, p.a_scale[m]);
    } else {
      store_out<KIND>(p, m, n, 0.f, v, p.a_scale[m]);
    }
  }
}

}  // namespace w4
