// Prefill-side kernel (M > 16): C[M,N] = A[M,K] x W[N,K]^T with INT8
// activations and 4-bit (or 2-bit ternary) weights on the CDNA4 INT8 matrix
// cores.
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
// Block: 256 threads = 4 waves in a 2 (m) x 2 (n) grid, block tile
// BM = 128 rows x BN = 16 * NTILES columns, wave tile 64 x 8*NTILES.
// Blocks are mapped so that each of the 8 XCDs works on a contiguous range of
// weight columns (its slice of W stays in that XCD's L2 while all m blocks
// pass over it).
#pragma once

#include "gemv.hpp"

namespace w4 {

constexpr int GEMM_THREADS = 256;
constexpr int GEMM_BM = 128;

template <int KIND>
struct GemmTraits {
  static constexpr int TILE_K = KindTraits<KIND>::TILE_K;  // k per stage (one weight tile)
  static constexpr int KSTEPS = TILE_K / 64;               // MFMA k steps per lane quarter
  static constexpr int A_STRIDE = TILE_K + 16;             // padded LDS row (bytes)
  static constexpr int A_BYTES = GEMM_BM * A_STRIDE;
  static constexpr int A_CHUNKS = GEMM_BM * TILE_K / 16 / GEMM_THREADS;  // per thread
};

template <int KIND, int NTILES>
struct GemmShape {
  using G = GemmTraits<KIND>;
  static constexpr int W_BYTES = NTILES * TILE_BYTES;
  static constexpr int STAGE = G::A_BYTES + W_BYTES;
  static constexpr int W_CHUNKS = NTILES * 64 / GEMM_THREADS;  // per thread
  static constexpr int NTW = NTILES / 2;                        // n subtiles per wave
};

struct GemmGrid {
  int mblocks, nblocks, tiles, ksplit, kts, per_xcd;
};

// unpack one 16-byte weight fragment into KSTEPS int8 MFMA operands
template <int KIND>
__device__ __forceinline__ void unpack_frag(const u4 w, i4 (&bf)[GemmTraits<KIND>::KSTEPS]) {
  if constexpr (KIND == KIND_W4A8) {
    bf[0] = unpack_w4_i8(w[0], w[1]);
    bf[1] = unpack_w4_i8(w[2], w[3]);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) bf[j] = unpack_w2_i8(w[j]);
  }
}

template <int KIND, int NTILES>
__global__ __launch_bounds__(GEMM_THREADS) void k_gemm(const MMParams p, const GemmGrid gg) {
  using G = GemmTraits<KIND>;
  using S = GemmShape<KIND, NTILES>;
  constexpr int TK = G::TILE_K;
  constexpr int J = G::KSTEPS;
  constexpr int NTW = S::NTW;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  // ---- block -> (m block, n block, k split) with XCD-contiguous n ranges --
  const int id = blockIdx.x;
  const int xcd = id & 7, local = id >> 3;
  const int tix = xcd * gg.per_xcd + local;          // n-major tile order
  if (local >= gg.per_xcd || tix >= gg.tiles) return;
  const int nb = tix / gg.mblocks;
  const int mb = tix - nb * gg.mblocks;
  const int kz = blockIdx.y;
  const int kb = kz * gg.kts;
  const int ke = min(p.KT, kb + gg.kts);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int r = lane & 15, b = lane >> 4;
  const int m0 = mb * GEMM_BM;
  const int t0 = nb * NTILES;                        // first n tile of the block

  const int8_t* A = reinterpret_cast<const int8_t*>(p.A);

  // ---- global -> register staging of one k tile ---------------------------
  u4 ra[G::A_CHUNKS];
  u4 rw[S::W_CHUNKS];
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < G::A_CHUNKS; ++i) {
      const int c = tid + i * GEMM_THREADS;          // chunk in the BM x TK tile
      const int row = c / (TK / 16), col = c % (TK / 16);
      const int gm = min(m0 + row, p.M - 1);
      const int gk = min(kt * TK + col * 16, p.K - 16);
      ra[i] = *reinterpret_cast<const u4*>(A + (size_t)gm * p.K + gk);
    }
#pragma unroll
    for (int i = 0; i < S::W_CHUNKS; ++i) {
      const int c = tid + i * GEMM_THREADS;          // chunk among NTILES x 64
      const int t = min(t0 + (c >> 6), p.NT - 1);
      rw[i] = __builtin_nontemporal_load(reinterpret_cast<const u4*>(
          p.Wt + ((size_t)t * p.KT + kt) * TILE_BYTES + (c & 63) * 16));
    }
  };
  auto sstore = [&](int kt, int buf) {
    uint8_t* sa = smem + buf * S::STAGE;
    uint8_t* sw = sa + G::A_BYTES;
#pragma unroll
    for (int i = 0; i < G::A_CHUNKS; ++i) {
      const int c = tid + i * GEMM_THREADS;
      const int row = c / (TK / 16), col = c % (TK / 16);
      u4 v = ra[i];
      if (kt * TK + col * 16 >= p.K) v = u4{0u, 0u, 0u, 0u};   // k tail
      *reinterpret_cast<u4*>(sa + row * G::A_STRIDE + col * 16) = v;
    }
#pragma unroll
    for (int i = 0; i < S::W_CHUNKS; ++i) {
      const int c = tid + i * GEMM_THREADS;
      *reinterpret_cast<u4*>(sw + c * 16) = rw[i];
    }
  };

  i4 acc[4][NTW];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int t = 0; t < NTW; ++t) acc[i][t] = i4{0, 0, 0, 0};

  if (kb < ke) {
    gload(kb);
    sstore(kb, 0);
  }
  __syncthreads();

  for (int kt = kb; kt < ke; ++kt) {
    const int buf = (kt - kb) & 1;
    const bool more = kt + 1 < ke;
    if (more) gload(kt + 1);

    const uint8_t* sa = smem + buf * S::STAGE;
    const uint8_t* sw = sa + G::A_BYTES;
    // activation fragments of this wave: 4 m subtiles x J k steps
    i4 af[4][J];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < J; ++j)
        af[i][j] = *reinterpret_cast<const i4*>(sa + (64 * wm + 16 * i + r) * G::A_STRIDE +
                                                (TK / 4) * b + 16 * j);
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      const u4 w = *reinterpret_cast<const u4*>(sw + (wn * NTW + t) * TILE_BYTES + lane * 16);
      i4 bf[J];
      unpack_frag<KIND>(w, bf);
#pragma unroll
      for (int j = 0; j < J; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc[i][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[i][j], bf[j], acc[i][t], 0, 0, 0);
    }

    if (more) sstore(kt + 1, buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue -------------------------------------------------------------
  const int ncol0 = (t0 + wn * NTW) * 16 + r;
  if (gg.ksplit == 1) {
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      const int n = ncol0 + 16 * t;
      if (n >= p.N) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = m0 + 64 * wm + 16 * i + 4 * b + e;
          const int v = acc[i][t][e];
          if (m < p.M) store_out<KIND>(p, m, n, 0.f, v);
        }
    }
    return;
  }

  // split K: exact INT32 partial sums, the last block of the tile finishes
  int32_t* part = reinterpret_cast<int32_t*>(p.partials);
  const size_t plane = (size_t)p.M * p.N;
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    const int n = ncol0 + 16 * t;
    if (n >= p.N) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = m0 + 64 * wm + 16 * i + 4 * b + e;
        const int v = acc[i][t][e];
        if (m < p.M) part[(size_t)kz * plane + (size_t)m * p.N + n] = v;
      }
  }
  __threadfence();
  __syncthreads();
  __shared__ int last;
  if (tid == 0) last = atomicAdd(&p.counters[tix], 1u) == (unsigned)(gg.ksplit - 1);
  __syncthreads();
  if (!last) return;
  __threadfence();
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    const int n = ncol0 + 16 * t;
    if (n >= p.N) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = m0 + 64 * wm + 16 * i + 4 * b + e;
        if (m >= p.M) continue;
        int s = 0;
        for (int z = 0; z < gg.ksplit; ++z) s += part[(size_t)z * plane + (size_t)m * p.N + n];
        store_out<KIND>(p, m, n, 0.f, s);
      }
  }
  if (tid == 0) p.counters[tix] = 0u;
}

// ---------------------------------------------------------------------------
// planning (host)
// ---------------------------------------------------------------------------
inline bool use_gemm(int kind, int M) { return kind != KIND_W4A16 && M > 16; }

inline int gemm_ntiles(int N) { return N >= 4096 ? 16 : 8; }

inline GemmGrid gemm_grid(int kind, int M, int N, int K) {
  const Geometry g = geometry(kind == KIND_W2A8 ? W4_LAYOUT_W2A8 : W4_LAYOUT_W4A8, N, K);
  GemmGrid gg{};
  const int nt = gemm_ntiles(N);
  gg.mblocks = ceil_div(M, GEMM_BM);
  gg.nblocks = ceil_div(g.NT, nt);
  gg.tiles = gg.mblocks * gg.nblocks;
  int ks = 1;
  while (gg.tiles * ks < 256 && ceil_div(g.KT, ks * 2) >= 2) ks *= 2;
  gg.kts = ceil_div(g.KT, ks);
  gg.ksplit = ceil_div(g.KT, gg.kts);
  gg.per_xcd = ceil_div(gg.tiles, 8);
  return gg;
}

inline size_t gemm_workspace_bytes(int kind, int M, int N, int K) {
  const GemmGrid gg = gemm_grid(kind, M, N, K);
  if (gg.ksplit == 1) return 0;
  const size_t counters = ((size_t)gg.tiles * sizeof(unsigned) + 255) & ~(size_t)255;
  return counters + (size_t)gg.ksplit * M * N * sizeof(int32_t);
}

template <int KIND, int NTILES>
int launch_gemm_t(MMParams p, const GemmGrid& gg, void* ws, hipStream_t stream) {
  using S = GemmShape<KIND, NTILES>;
  p.counters = reinterpret_cast<unsigned*>(ws);
  const size_t counters = ((size_t)gg.tiles * sizeof(unsigned) + 255) & ~(size_t)255;
  p.partials = ws ? reinterpret_cast<uint8_t*>(ws) + counters : nullptr;
  const dim3 grid(gg.per_xcd * 8, gg.ksplit);
  allow_smem((const void*)&k_gemm<KIND, NTILES>, 2 * S::STAGE);
  hipLaunchKernelGGL((k_gemm<KIND, NTILES>), grid, dim3(GEMM_THREADS), 2 * S::STAGE, stream, p,
                     gg);
  return launch_status();
}

template <int KIND>
int launch_gemm(const MMParams& p, void* ws, hipStream_t stream) {
  if constexpr (KIND == KIND_W4A16) {
    return W4_ERR_ARG;
  } else {
    const GemmGrid gg = gemm_grid(KIND, p.M, p.N, p.K);
    if (gemm_ntiles(p.N) == 16) return launch_gemm_t<KIND, 16>(p, gg, ws, stream);
    return launch_gemm_t<KIND, 8>(p, gg, ws, stream);
  }
}

}  // namespace w4
