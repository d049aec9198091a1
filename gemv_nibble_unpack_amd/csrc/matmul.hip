// C-ABI matmul entry points: argument validation, launch planning, dispatch
// between the decode kernel (M <= 16) and the prefill GEMM kernel.

#include <algorithm>
#include <atomic>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <tuple>

#include "gemm.hpp"
#include "gemv.hpp"
#include "skinny.hpp"

namespace w4 {

constexpr int GEMV_WAVES = 8;             // decode block: 8 waves, or 16 for long k runs
constexpr int SPLIT_BELOW = 64;            // blocks below which K is split
constexpr int STAGE_MAX = 64 * 1024;       // activation bytes one block may stage

// The three ways a product can run. Every candidate computes the same
// result; they differ in how the work is cut into blocks.
enum PlanPath { PATH_DECODE = 0, PATH_SKINNY = 1, PATH_GEMM = 2 };

struct Candidate {
  int path;
  int ks;           // decode, skinny: requested k split (0: chosen from the grid size)
  GemmCfg cfg;      // gemm: block shape
  int mt;           // skinny: 16-row activation tiles per block (0 or 1: one, up to 4)
  int waves;        // decode: waves per block (0 or 8: eight, 16: sixteen)
};

struct Plan {
  bool gemm;        // prefill kernel instead of the decode kernel
  bool skinny;      // > 16 rows without enough GEMM tiles: 16 rows x 128 columns per block
  int mtb;          // skinny: 16-row activation tiles per block (1 to 4)
  GemmCfg cfg;      // gemm: block shape
  int ngroups;      // skinny: groups of 8 weight n-tiles
  bool staged;      // activation rows staged in LDS
  bool wst;         // staged per wave (each wave its own k range, no block barrier)
  int apw;          // wave staging: 16-byte loads per lane
  int ksplit, kts, mtiles, maxt, aper;
  int waves;        // decode: waves per block (8, or 16 with wave staging)
  bool m1;          // decode, W4A16, one row: the one-row offset scheme
  size_t smem;
  size_t counters_bytes, ws_bytes;
};

inline int kind_layout(int kind) {
  // the 2-bit weights serve INT8 and fp16 activations from one prepacked
  // layout; INT8 and FP8 weights share the byte-tile layout
  switch (kind) {
    case KIND_W4A8: return W4_LAYOUT_W4A8;
    case KIND_W4A16: return W4_LAYOUT_W4A16;
    case KIND_W8A8:
    case KIND_F8F8: return W4_LAYOUT_W8A8;
    default: return W4_LAYOUT_W2A8;
  }
}

// activation bytes per row per weight tile (the tile's k extent x element size)
inline int tile_rowb(int kind) {
  switch (kind) {
    case KIND_W4A16: return 256;
    case KIND_W4A8: return 128;
    case KIND_W2A16: return 512;
    case KIND_W8A8:
    case KIND_F8F8: return 64;
    default: return 256;
  }
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// The plan a candidate gives for one shape.
inline Plan plan_from(int kind, int M, int N, int K, const Candidate& c) {
  const Geometry g = geometry(kind_layout(kind), N, K);
  Plan P{};
  if (c.path == PATH_GEMM) {
    P.gemm = true;
    P.cfg = c.cfg;
    P.ksplit = gemm_grid(kind, M, N, K, c.cfg).ksplit;
    P.ws_bytes = gemm_workspace_bytes(kind, M, N, K, c.cfg);
    return P;
  }
  P.mtiles = ceil_div(M, 16);
  P.ngroups = ceil_div(g.NT, SKINNY_WAVES);
  if (c.path == PATH_SKINNY) {
    P.skinny = true;
    P.mtb = c.mt >= 2 && c.mt <= 4 ? c.mt : 1;
    P.mtiles = ceil_div(M, 16 * P.mtb);            // blocks of 16 mtb rows
    // k split: one counter per (row tile, column group)
    const int ks = c.ks > 1 && P.mtiles * P.ngroups <= WS_COUNTER_SLOTS ? c.ks : 1;
    P.kts = ceil_div(g.KT, ks);
    P.ksplit = ceil_div(g.KT, P.kts);
    if (P.ksplit > 1) {
      P.counters_bytes = WS_COUNTERS;
      P.ws_bytes = WS_COUNTERS + (size_t)P.mtiles * P.ksplit * P.ngroups * SKINNY_WAVES * 256 *
                                     P.mtb * 4;
    }
    return P;
  }
  const int rows = M < 16 ? M : 16;
  const int blocks = g.NT * P.mtiles;
  const int trb = tile_rowb(kind);
  const int W = c.waves == 16 ? 16 : c.waves == 4 ? 4 : GEMV_WAVES;
  P.waves = W;
  int ks = g.NT * P.mtiles <= WS_COUNTER_SLOTS ? c.ks : 1;  // one counter per block slot
  if (ks <= 0) {
    // split K across blocks only when the grid would leave most CUs idle,
    // keeping a tile per wave (larger grids gain little or lose from the
    // partial-sum round trip; the plan table can pin a split per shape)
    ks = 1;
    while (blocks * ks < SPLIT_BELOW && ceil_div(g.KT, ks * 2) >= W) ks *= 2;
  }
  // W4A16 cuts K on even tiles: every wave's run starts on an even tile, and
  // the scales and zeros of its tiles come in whole quads of groups
  const bool pairs = kind == KIND_W4A16;
  P.kts = pairs ? 2 * ceil_div(ceil_div(g.KT, 2), ks) : ceil_div(g.KT, ks);
  P.ksplit = ceil_div(g.KT, P.kts);
  const int per = pairs ? 2 * ceil_div(ceil_div(P.kts, 2), W) : ceil_div(P.kts, W);
  // (six tiles: W4A16 runs of 5..6 tiles at sixteen waves, e.g. K = 11008,
  // which eight slots would pad with two dead loads per wave)
  P.maxt = per <= 2 && W == 16                               ? 2
           : per <= 4                                        ? 4
           : per <= 6 && W == 16 && kind == KIND_W4A16       ? 6
           : per <= 8                                        ? 8
                                                             : 16;
  // stage the block's activation rows in LDS when they fit, else each lane
  // streams its own fragments from L2
  P.staged = (size_t)rows * P.kts * trb <= (size_t)STAGE_MAX;
  const int chunks = ceil_div(rows * P.kts * trb, 16);
  const int aper = ceil_div(chunks, W * 64);
  P.aper = aper <= 1 ? 1 : aper <= 2 ? 2 : aper <= 4 ? 4 : 8;
  // small per-wave ranges (up to 4 loads per lane) are staged by each wave
  // for itself: a wave then starts on its first tile without waiting for the
  // slowest wave of the block
  const int wchunks = rows * per * trb / 16;
  P.wst = P.staged && wchunks <= 4 * 64;
  // sixteen waves run with wave staging (up to 8 tiles per wave) or without
  // staging (up to 4, and not for fp16 x 2-bit, whose 8 fragment loads per
  // tile would not fit the activation ring in 128 registers); otherwise the
  // plan is the eight-wave one
  if (W == 16 && ((P.staged && !P.wst) || per > 8 ||
                  (!P.staged && (per > 4 || kind == KIND_W2A16))))
    return plan_from(kind, M, N, K, Candidate{PATH_DECODE, c.ks, {}, 0, 8});
  // four waves run only with wave staging
  if (W == 4 && !P.wst) return plan_from(kind, M, N, K, Candidate{PATH_DECODE, c.ks, {}, 0, 8});
  P.apw = wchunks <= 64 ? 1 : wchunks <= 128 ? 2 : 4;
  // one row, staged per wave in one pass
  P.m1 = kind == KIND_W4A16 && M == 1 && P.wst && per <= P.maxt;
  const size_t block_stage = P.staged ? (size_t)rows * (P.kts * trb + 16) : 0;
  const size_t wave_stage = P.wst ? (size_t)W * rows * (per * trb + 16) : 0;
  P.smem = std::max({block_stage, wave_stage, (size_t)W * 1024});
  if (P.ksplit > 1) {
    P.counters_bytes = WS_COUNTERS;
    P.ws_bytes = WS_COUNTERS + (size_t)P.mtiles * P.ksplit * g.NT * 256 * 4;
  }
  return P;
}

constexpr int CAND_MAX_BLOCKS = 1024;      // k splits tried up to this many blocks
constexpr size_t REREAD_MAX = 64ull << 20;   // activation bytes the decode kernel may re-read
constexpr int SKINNY_RESIDENT = 512;         // skinny blocks resident at once (two per CU)
constexpr int SKINNY_TILES = 12;             // k tiles per block aimed at by a skinny split

// The built-in choice: the prefill GEMM when it has enough tiles, the skinny
// kernel when several activation tiles can share staged rows across enough
// blocks, else the decode kernel with its own k split -- unless the decode
// kernel cannot stage the rows in LDS and its blocks would re-read more than
// 64 MiB of them from L2 (e.g. 16 fp16 rows at N = 11008, K = 4096, or at
// N = 4096, K = 11008: 90 MB); then the skinny kernel, which reads them once
// per 8 n-tiles, runs with a k split that leaves about 12 k tiles per block
// (W4A16 M=16 on MI355X: 17.2 -> 13.8 us and 21.2 -> 13.8 us).
inline Candidate heuristic(int kind, int M, int N, int K) {
  if (use_gemm(kind, M, N)) return Candidate{PATH_GEMM, 0, gemm_cfg(kind, M, N)};
  const Geometry g = geometry(kind_layout(kind), N, K);
  const int mtiles = ceil_div(M, 16);
  const int ngroups = ceil_div(g.NT, SKINNY_WAVES);
  // more row tiles per block once one-tile blocks would need more than the
  // 512 resident at two per CU: three where that leaves one block per CU at
  // most, else two (M=128 N=8640 K=3200 on MI355X: W2A8 13.8 -> 12.9 us,
  // W2A16 22.9 -> 19.6 us at three; four tiles, 136 blocks, 15.4 and 23.6)
  if (mtiles > 1 && ngroups * mtiles >= SPLIT_BELOW) {
    // fp16 x 2-bit rows over 24 or more k tiles: two row tiles per block (the
    // crumb unpack, VALU-bound, is shared by both) and the power-of-two k
    // split nearest to 5 k tiles per block (M=128 N=3200 K=8640 on MI355X:
    // one-tile blocks 24.5 us, two-tile blocks split 4 / 7 ways 22.4 / 21.6)
    if (kind == KIND_W2A16 && g.KT >= 24) {
      const float want = (float)g.KT / 5.0f;
      int ks = 1;
      while (ks * 2 <= 64 && (float)(ks * 2) <= want * 1.41421356f) ks *= 2;
      const Candidate c{PATH_SKINNY, ks, {}, 2};
      const Plan pc = plan_from(kind, M, N, K, c);
      if (pc.ksplit > 1 && ngroups * ceil_div(M, 32) * pc.ksplit <= CAND_MAX_BLOCKS) return c;
    }
    if (ngroups * mtiles <= SKINNY_RESIDENT) return Candidate{PATH_SKINNY, 0, {}, 1};
    return Candidate{PATH_SKINNY, 0, {}, ngroups * ceil_div(M, 48) <= GEMM_CUS ? 3 : 2};
  }
  const int rows = M < 16 ? M : 16;
  const size_t row_bytes = (size_t)g.KT * tile_rowb(kind);
  if (mtiles == 1 && (size_t)rows * row_bytes > (size_t)STAGE_MAX &&
      (size_t)g.NT * rows * row_bytes > REREAD_MAX) {
    // nearest power of two to KT / 12
    const float want = (float)g.KT / SKINNY_TILES;
    int ks = 1;
    while (ks * 2 <= 64 && (float)(ks * 2) <= want * 1.41421356f) ks *= 2;
    return Candidate{PATH_SKINNY, ks, {}};
  }
  // Sixteen waves per block, each with half as long a k run, where the grid
  // needs no k split and either (a) one row of K >= 8192 is staged per wave
  // over one block per CU at most, or with more than 8 tiles per wave at
  // eight waves (whose 16 weight registers per lane would leave one block per
  // CU) (M=1 on MI355X: W4A16 N=4096 K=11008 9.46 -> 8.54 us, N=K=16384
  // 39.0 -> 33.7, W2A16 N=3200 K=8640 6.38 -> 5.79, W2A8 N=3200 K=8640
  // 4.78 -> 4.44; at K <= 4096, or more blocks of at most 8 tiles per wave,
  // eight waves are as fast or faster at M=1: N=28672 K=8192 26.2 vs 32.1),
  // or (b) 4 to 16 rows of K <= 4096 (W4A16 M=4 4096x4096 5.33 -> 5.15, M=4
  // N=11008 9.51 -> 8.97, M=16 4096x4096 8.22 -> 7.93)
  const Candidate wide{PATH_DECODE, 0, {}, 0, 16};
  const Plan pw = plan_from(kind, M, N, K, wide);
  const bool long_runs = ceil_div(g.KT, GEMV_WAVES) > 8;
  if (mtiles == 1 && g.NT >= SPLIT_BELOW && pw.waves == 16 && pw.ksplit == 1 &&
      ((K >= 8192 && (g.NT <= 256 || long_runs) && pw.wst) || (rows >= 4 && K <= 4096)))
    return wide;
  // Four waves per block, each with twice as long a k run, for one row of
  // INT8 or FP8 activations of K <= 4096 over 64..639 unsplit blocks (M=1 on
  // MI355X: W2A8 N=8640 K=3200 4.65 -> 4.42 us, N=K=3200 3.43 -> 3.34, W4A8
  // 4096x4096 4.31 -> 4.24, INT8 and FP8 weights 4096x4096 -1.3%; fp16
  // activations, or 688 blocks (W4A8 N=11008), lose 2..12%)
  const bool a8 = kind == KIND_W4A8 || kind == KIND_W2A8 || kind == KIND_W8A8 || kind == KIND_F8F8;
  const Candidate narrow{PATH_DECODE, 0, {}, 0, 4};
  if (a8 && rows == 1 && K <= 4096 && g.NT >= SPLIT_BELOW && g.NT < 640) {
    const Plan pn = plan_from(kind, M, N, K, narrow);
    if (pn.waves == 4 && pn.ksplit == 1) return narrow;
  }
  // up to 4 rows too long to stage in LDS at all: the smallest k split (up to
  // 1024 blocks) that lets every wave stage its own range (M=4, N=4096,
  // K=11008 on MI355X: 13.27 -> 11.77 us at 4 splits; 2 splits, staged per
  // block, took 14.69). Rows that the block can stage stay unsplit (M=1,
  // N=8192, K=28672: 33.9 us unsplit, 39.5 at 2 splits).
  if (rows <= 4 && !plan_from(kind, M, N, K, Candidate{PATH_DECODE, 0, {}}).staged) {
    for (int ks = 2; ks <= 8 && g.NT * ks <= CAND_MAX_BLOCKS; ks *= 2) {
      const Candidate c{PATH_DECODE, ks, {}};
      if (plan_from(kind, M, N, K, c).wst) return c;
    }
  }
  return Candidate{PATH_DECODE, 0, {}};
}

constexpr int MAX_CANDIDATES = 64;

// Every plan that may run the shape, in a fixed order: the decode kernel at
// each distinct k split that keeps a tile per wave (each followed by its
// sixteen-wave form where that exists), the skinny kernel, then (INT8
// activations, more than 16 rows) each GEMM block shape.
inline int candidates(int kind, int M, int N, int K, Candidate* out) {
  const Geometry g = geometry(kind_layout(kind), N, K);
  const int blocks = g.NT * ceil_div(M, 16);
  int n = 0, last = 0;
  for (int ks = 1; ks <= 64; ks *= 2) {
    if (ks > 1 && (ceil_div(g.KT, ks) < GEMV_WAVES || blocks * ks > CAND_MAX_BLOCKS)) break;
    const int eff = plan_from(kind, M, N, K, Candidate{PATH_DECODE, ks, {}}).ksplit;
    if (eff == last) continue;
    last = eff;
    out[n++] = Candidate{PATH_DECODE, ks, {}};
    // the same split with four and with sixteen waves per block, where those
    // plans exist
    const Candidate narrow{PATH_DECODE, ks, {}, 0, 4};
    if (plan_from(kind, M, N, K, narrow).waves == 4) out[n++] = narrow;
    const Candidate wide{PATH_DECODE, ks, {}, 0, 16};
    if (plan_from(kind, M, N, K, wide).waves == 16) out[n++] = wide;
  }
  // the skinny kernel (one, and above 16 rows also two, row tiles per block),
  // whole K and at each distinct k split up to the same block count
  for (int mt = 1; mt <= std::min(4, ceil_div(M, 16)); ++mt) {
    const int sblocks = ceil_div(g.NT, SKINNY_WAVES) * ceil_div(M, 16 * mt);
    last = 0;
    for (int ks = 1; ks <= 64; ks *= 2) {
      if (ks > 1 && (ceil_div(g.KT, ks) < 2 || sblocks * ks > CAND_MAX_BLOCKS)) break;
      const int eff = ceil_div(g.KT, ceil_div(g.KT, ks));
      if (eff == last) continue;
      last = eff;
      out[n++] = Candidate{PATH_SKINNY, ks, {}, mt};
    }
  }
  if (M > 16 && kind == KIND_W4A8) {
    out[n++] = Candidate{PATH_GEMM, 0, GemmCfg{16, 2}};
    out[n++] = Candidate{PATH_GEMM, 0, GemmCfg{22, 2}};
    out[n++] = Candidate{PATH_GEMM, 0, GemmCfg{22, 4}};
  } else if (M > 16 && kind == KIND_W4A16) {
    // fp16 activations: 128 x 256, 128 x 352 and 128 x 384 blocks, whole K
    out[n++] = Candidate{PATH_GEMM, 0, GemmCfg{16, 2}};
    out[n++] = Candidate{PATH_GEMM, 0, GemmCfg{22, 2}};
    out[n++] = Candidate{PATH_GEMM, 0, GemmCfg{24, 2}};
  } else if (M > 16 && kind == KIND_F8F8) {
    // FP8: 128 x 128 blocks over the whole K (float32 sums are not split)
    out[n++] = Candidate{PATH_GEMM, 0, GemmCfg{8, 2}};
  } else if (M > 16 && (kind == KIND_W2A8 || kind == KIND_W8A8)) {
    // 128 x 128 blocks, whole K and at each distinct k split up to the same
    // block count
    const int tiles = gemm_tiles(M, N, GemmCfg{8, 2});
    last = 0;
    for (int ks = 1; ks <= 64; ks *= 2) {
      if (ks > 1 && (ceil_div(g.KT, ks) < 2 || tiles * ks > CAND_MAX_BLOCKS)) break;
      const int eff = gemm_grid(kind, M, N, K, GemmCfg{8, 2, ks}).ksplit;
      if (eff == last) continue;
      last = eff;
      out[n++] = Candidate{PATH_GEMM, 0, GemmCfg{8, 2, ks}};
    }
  }
  return n;
}

inline bool same_plan(const Plan& a, const Plan& b) {
  if (a.gemm != b.gemm || a.skinny != b.skinny) return false;
  if (a.gemm) return a.cfg.ntiles == b.cfg.ntiles && a.cfg.wm == b.cfg.wm && a.ksplit == b.ksplit;
  if (a.skinny && a.mtb != b.mtb) return false;
  if (!a.skinny && a.waves != b.waves) return false;
  return a.ksplit == b.ksplit;
}

// Plans pinned per shape (w4_plan_pin); a shape without one takes the
// built-in choice. One table per process, shared by all devices.
typedef std::tuple<int, int, int, int> ShapeKey;
inline std::mutex& pin_mutex() {
  static std::mutex m;
  return m;
}
inline std::map<ShapeKey, Candidate>& pin_table() {
  static std::map<ShapeKey, Candidate> t;
  return t;
}
inline std::atomic<int>& pin_count() {
  static std::atomic<int> c{0};
  return c;
}

inline Candidate chosen(int kind, int M, int N, int K) {
  if (pin_count().load(std::memory_order_acquire) > 0) {
    std::lock_guard<std::mutex> lock(pin_mutex());
    const auto it = pin_table().find(ShapeKey{kind, M, N, K});
    if (it != pin_table().end()) return it->second;
  }
  return heuristic(kind, M, N, K);
}

// Deterministic in (kind, M, N, K) and the pin table: w4_workspace_bytes and
// the launch agree as long as no pin changes in between.
inline Plan make_plan(int kind, int M, int N, int K) {
  return plan_from(kind, M, N, K, chosen(kind, M, N, K));
}

// Chunk slots per lane the fused-quantization prologue needs for a block of
// `rows` activation rows (see k_gemv), or 0 when more than 8 would be needed.
inline int fq_slots(int rows, int K) {
  const int rpw = rows > 8 ? 2 : 1;
  const int g = rows > 4 ? 1 : rows > 2 ? 2 : rows > 1 ? 4 : 8;
  const int need = rpw * ceil_div(K / 8, 64 * g);
  return need <= 2 ? 2 : need <= 8 ? 8 : 0;
}

// Launch one decode-kernel instance: the fields its first loads depend on go
// as leading scalar arguments, which the build preloads into SGPRs.
template <typename Kern>
inline void gemv_go(Kern kern, dim3 grid, dim3 block, size_t smem, hipStream_t stream,
                    const MMParams& p) {
  allow_smem((const void*)kern, smem);
  hipLaunchKernelGGL(kern, grid, block, smem, stream, p.Wt, p.A, p.St, p.Zt, p.M, p.K, p.KT,
                     p.KQ, p.kts, p);
}

template <int KIND, int WAVES, int MAXT>
int launch_gemv_m(const Plan& P, const MMParams& p, hipStream_t stream, int fq = 0, int fqc = 0) {
  // x enumerates (n tile, m tile) pairs so that the m tiles of one n tile land
  // on the same XCD (blocks are dealt to the 8 XCDs round-robin by id)
  const int nblk = P.mtiles == 1 ? p.NT : ceil_div(p.NT * P.mtiles, 8) * 8;
  const dim3 grid(nblk, P.ksplit, 1);
  const dim3 block(WAVES * 64);
  // wave staging; for W4A16 at one row the one-row offset scheme (the
  // planner sets m1 only for plans it fits)
  auto wcase = [&](auto aper) {
    constexpr int A = decltype(aper)::value;
    if constexpr (KIND == KIND_W4A16) {
      if (P.m1) {
        gemv_go(&k_gemv<KIND, WAVES, MAXT, A, true, 0, 1, true, true>, grid, block, P.smem,
                stream, p);
        return;
      }
    }
    gemv_go(&k_gemv<KIND, WAVES, MAXT, A, true, 0, 1, true>, grid, block, P.smem, stream, p);
  };
  using A1 = std::integral_constant<int, 1>;
  using A2 = std::integral_constant<int, 2>;
  using A4 = std::integral_constant<int, 4>;
  if constexpr (WAVES != 8) {
    // sixteen- and four-wave plans stage per wave or not at all, and never
    // quantize in the prologue (the planner guarantees both)
    if (fq || (P.staged && !P.wst)) return W4_ERR_ARG;
    if (!P.staged) {
      if constexpr (WAVES == 16 && MAXT <= 4 && KIND != KIND_W2A16) {
        gemv_go(&k_gemv<KIND, WAVES, MAXT, 1, false>, grid, block, P.smem, stream, p);
      } else {
        return W4_ERR_ARG;
      }
    } else if (P.apw == 1) {
      wcase(A1{});
    } else if (P.apw == 2) {
      wcase(A2{});
    } else {
      wcase(A4{});
    }
    return launch_status();
  } else {
    if constexpr (KIND == KIND_W4A8 || KIND == KIND_W2A8) {
      if (fq) {
        if (fq == 1 && fqc == 2) gemv_go(&k_gemv<KIND, WAVES, MAXT, 1, true, 1, 2>, grid, block, P.smem, stream, p);
        else if (fq == 1) gemv_go(&k_gemv<KIND, WAVES, MAXT, 1, true, 1, 8>, grid, block, P.smem, stream, p);
        else if (fqc == 2) gemv_go(&k_gemv<KIND, WAVES, MAXT, 1, true, 2, 2>, grid, block, P.smem, stream, p);
        else gemv_go(&k_gemv<KIND, WAVES, MAXT, 1, true, 2, 8>, grid, block, P.smem, stream, p);
        return launch_status();
      }
    }
    if (!P.staged) {
      gemv_go(&k_gemv<KIND, WAVES, MAXT, 1, false>, grid, block, P.smem, stream, p);
    } else if (P.wst) {
      if (P.apw == 1) wcase(A1{});
      else if (P.apw == 2) wcase(A2{});
      else wcase(A4{});
    } else {
      switch (P.aper) {
        case 1: gemv_go(&k_gemv<KIND, WAVES, MAXT, 1, true>, grid, block, P.smem, stream, p); break;
        case 2: gemv_go(&k_gemv<KIND, WAVES, MAXT, 2, true>, grid, block, P.smem, stream, p); break;
        case 4: gemv_go(&k_gemv<KIND, WAVES, MAXT, 4, true>, grid, block, P.smem, stream, p); break;
        default: gemv_go(&k_gemv<KIND, WAVES, MAXT, 8, true>, grid, block, P.smem, stream, p); break;
      }
    }
    return launch_status();
  }
}

template <int KIND>
int launch_gemv(const Plan& P, MMParams p, void* ws, hipStream_t stream, int fq = 0, int fqc = 0) {
  p.ksplit = P.ksplit;
  p.kts = P.kts;
  p.counters = reinterpret_cast<unsigned*>(ws);
  p.partials = ws ? reinterpret_cast<uint8_t*>(ws) + P.counters_bytes : nullptr;
  if (P.waves == 4) {
    if (P.maxt == 4) return launch_gemv_m<KIND, 4, 4>(P, p, stream, fq, fqc);
    if (P.maxt == 8) return launch_gemv_m<KIND, 4, 8>(P, p, stream, fq, fqc);
    return launch_gemv_m<KIND, 4, 16>(P, p, stream, fq, fqc);
  }
  if (P.waves == 16) {
    if (P.maxt == 2) return launch_gemv_m<KIND, 16, 2>(P, p, stream, fq, fqc);
    if (P.maxt == 4) return launch_gemv_m<KIND, 16, 4>(P, p, stream, fq, fqc);
    if constexpr (KIND == KIND_W4A16) {
      if (P.maxt == 6) return launch_gemv_m<KIND, 16, 6>(P, p, stream, fq, fqc);
    }
    return launch_gemv_m<KIND, 16, 8>(P, p, stream, fq, fqc);
  }
  if (P.maxt == 4) return launch_gemv_m<KIND, 8, 4>(P, p, stream, fq, fqc);
  if (P.maxt == 8) return launch_gemv_m<KIND, 8, 8>(P, p, stream, fq, fqc);
  return launch_gemv_m<KIND, 8, 16>(P, p, stream, fq, fqc);
}

template <int KIND>
int launch_skinny(const Plan& P, MMParams p, void* ws, hipStream_t stream) {
  p.ksplit = P.ksplit;
  p.kts = P.kts;
  p.counters = reinterpret_cast<unsigned*>(ws);
  p.partials = ws ? reinterpret_cast<uint8_t*>(ws) + P.counters_bytes : nullptr;
  const dim3 grid(ceil_div(P.ngroups * P.mtiles, 8) * 8, P.ksplit);
#define W4_SKINNY(SPLIT, MTB)                                                               \
  do {                                                                                      \
    const size_t smem = skinny_smem<KIND, MTB>();                                           \
    allow_smem((const void*)&k_skinny<KIND, 8, SPLIT, MTB>, smem);                          \
    hipLaunchKernelGGL((k_skinny<KIND, 8, SPLIT, MTB>), grid, dim3(SKINNY_THREADS), smem,   \
                       stream, p.Wt, p.A, p.St, p.Zt, p.M, p.K, p.NT, p.kts, P.ngroups,     \
                       (int)(grid.x / 8), p);                                               \
  } while (0)
  if (P.mtb == 4) {
    if (P.ksplit > 1) W4_SKINNY(true, 4);
    else W4_SKINNY(false, 4);
  } else if (P.mtb == 3) {
    if (P.ksplit > 1) W4_SKINNY(true, 3);
    else W4_SKINNY(false, 3);
  } else if (P.mtb == 2) {
    if (P.ksplit > 1) W4_SKINNY(true, 2);
    else W4_SKINNY(false, 2);
  } else {
    if (P.ksplit > 1) W4_SKINNY(true, 1);
    else W4_SKINNY(false, 1);
  }
#undef W4_SKINNY
  return launch_status();
}

template <int KIND>
int run(MMParams p, void* ws, size_t ws_bytes, hipStream_t stream) {
  const Plan P = make_plan(KIND, p.M, p.N, p.K);
  if (P.ws_bytes) {
    if (!ws || ws_bytes < P.ws_bytes) return W4_ERR_WORKSPACE;
    if (!aligned(ws, 16)) return W4_ERR_ALIGN;
  }
  const Geometry g = geometry(kind_layout(KIND), p.N, p.K);
  p.NT = g.NT;
  p.KT = g.KT;
  p.KQ = g.KQ;
  if (P.gemm) return launch_gemm<KIND>(p, P.cfg, ws, stream);
  if (P.skinny) return launch_skinny<KIND>(P, p, ws, stream);
  return launch_gemv<KIND>(P, p, ws, stream);
}

inline int check_common(int M, int N, int K, int kmult) {
  if (M < 0 || N < 1 || K < kmult || K > W4_MAX_K || K % kmult) return W4_ERR_SHAPE;
  return W4_OK;
}

inline bool out_aligned(const void* C, int out_dtype) {
  return aligned(C, out_dtype == W4_OUT_F16 ? 2 : 4);
}

}  // namespace w4

using namespace w4;

extern "C" size_t w4_workspace_bytes(int layout, int M, int N, int K) {
  int kind;
  if (layout == W4_LAYOUT_W4A8) kind = KIND_W4A8;
  else if (layout == W4_LAYOUT_W4A16) kind = KIND_W4A16;
  else if (layout == W4_LAYOUT_W2A8) kind = KIND_W2A8;
  else if (layout == W4_LAYOUT_W8A8) kind = KIND_W8A8;
  else return 0;
  if (check_common(M, N, K, kind == KIND_W4A16 ? W4_GROUP_SIZE : 16) != W4_OK || M == 0) return 0;
  return make_plan(kind, M, N, K).ws_bytes;
}

static int a8_common(int kind, const int8_t* Aq, const float* a_scale, const uint8_t* Wp,
                     const void* scale, const uint16_t* bias, void* C, int out_dtype, int M, int N,
                     int K, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (out_dtype != W4_OUT_F16 && out_dtype != W4_OUT_F32 && out_dtype != W4_OUT_I32)
    return W4_ERR_ARG;
  const int st = check_common(M, N, K, 16);
  if (st != W4_OK) return st;
  if (M == 0) return W4_OK;
  if (!Aq || !a_scale || !Wp || !scale || !C) return W4_ERR_NULL;
  if (!aligned(Aq, 16) || !aligned(Wp, 16) || !aligned(a_scale, 4) || !out_aligned(C, out_dtype) ||
      (bias && !aligned(bias, 2)) || !aligned(scale, kind == KIND_W4A8 ? 4 : 2))
    return W4_ERR_ALIGN;
  MMParams p{};
  p.A = Aq;
  p.a_scale = a_scale;
  p.Wt = Wp;
  p.w_scale = kind == KIND_W4A8 ? (const float*)scale : nullptr;
  p.w_scale16 = kind == KIND_W2A8 ? (const uint16_t*)scale : nullptr;
  p.bias = out_dtype == W4_OUT_I32 ? nullptr : bias;
  p.C = C;
  p.out_dtype = out_dtype;
  p.M = M;
  p.N = N;
  p.K = K;
  return kind == KIND_W4A8 ? run<KIND_W4A8>(p, ws, ws_bytes, stream)
                           : run<KIND_W2A8>(p, ws, ws_bytes, stream);
}

extern "C" int w4a8_gemm(const int8_t* Aq, const float* a_scale, const uint8_t* Wp,
                         const float* w_scale, const uint16_t* bias, void* C, int out_dtype, int M,
                         int N, int K, void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
  return a8_common(KIND_W4A8, Aq, a_scale, Wp, w_scale, bias, C, out_dtype, M, N, K, workspace,
                   workspace_bytes, stream);
}

extern "C" int w2a8_gemm(const int8_t* Aq, const float* a_scale, const uint8_t* Wp,
                         const uint16_t* w_scale16, const uint16_t* bias, void* C, int out_dtype,
                         int M, int N, int K, void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
  return a8_common(KIND_W2A8, Aq, a_scale, Wp, w_scale16, bias, C, out_dtype, M, N, K, workspace,
                   workspace_bytes, stream);
}

extern "C" int w4a16_gemm(const uint16_t* A, const uint8_t* Wp, int group_size,
                          const uint16_t* bias, uint16_t* C, int M, int N, int K, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  if (group_size != W4_GROUP_SIZE) return W4_ERR_ARG;
  const int st = check_common(M, N, K, W4_GROUP_SIZE);
  if (st != W4_OK) return st;
  if (M == 0) return W4_OK;
  if (!A || !Wp || !C) return W4_ERR_NULL;
  if (!aligned(A, 16) || !aligned(Wp, 16) || !aligned(C, 2) || (bias && !aligned(bias, 2)))
    return W4_ERR_ALIGN;
  const Geometry g = geometry(W4_LAYOUT_W4A16, N, K);
  MMParams p{};
  p.A = A;
  p.Wt = Wp;
  p.St = reinterpret_cast<const uint16_t*>(Wp + g.s_off);
  p.Zt = Wp + g.z_off;
  p.bias = bias;
  p.C = C;
  p.out_dtype = W4_OUT_F16;
  p.M = M;
  p.N = N;
  p.K = K;
  return run<KIND_W4A16>(p, workspace, workspace_bytes, stream);
}

// ---------------------------------------------------------------------------
// fused activation quantization: quantize_a8 + w4a8_gemm / w2a8_gemm in one
// call. Decode shapes whose activation rows fit the block's LDS staging run
// one kernel that quantizes in its prologue; everything else (prefill GEMM
// and skinny shapes, decode rows too long to stage) quantizes into the
// workspace with quantize_a8 first and then runs the A8 matmul.
// ---------------------------------------------------------------------------
namespace w4 {

struct FusedPlan {
  Plan P;
  int fqc;            // decode prologue slots per lane (0: not that form)
  size_t q_off;       // offset of the quantized rows and their scales
  size_t ws_bytes;    // total workspace
};

// Quantized rows in the workspace: the matmul's own workspace (counters,
// partial sums) keeps offset 0 and the rows follow it, past the counter area
// even when the matmul does not split, so the counters of every call stay
// where they are in every other call.
inline FusedPlan fused_plan(int kind, int M, int N, int K) {
  FusedPlan F{};
  F.P = make_plan(kind, M, N, K);
  // the quantizing prologue runs in eight-wave blocks: a sixteen-wave plan
  // becomes the eight-wave plan of the same split
  if (!F.P.gemm && !F.P.skinny && F.P.waves != 8)
    F.P = plan_from(kind, M, N, K, Candidate{PATH_DECODE, F.P.ksplit, {}, 0, 8});
  F.fqc = (!F.P.gemm && !F.P.skinny && F.P.staged) ? fq_slots(M < 16 ? M : 16, K) : 0;
  if (F.fqc) {
    F.ws_bytes = F.P.ws_bytes;
  } else {
    F.q_off = align256(std::max(F.P.ws_bytes, WS_COUNTERS));
    F.ws_bytes = F.q_off + align256((size_t)M * K) + align256((size_t)M * sizeof(float));
  }
  return F;
}

}  // namespace w4

extern "C" size_t w4_fused_act_workspace_bytes(int layout, int M, int N, int K) {
  if (layout != W4_LAYOUT_W4A8 && layout != W4_LAYOUT_W2A8) return 0;
  if (check_common(M, N, K, 16) != W4_OK || M == 0) return 0;
  return fused_plan(layout == W4_LAYOUT_W4A8 ? KIND_W4A8 : KIND_W2A8, M, N, K).ws_bytes;
}

extern "C" int quantize_a8(const void* A, int in_dtype, int M, int K, int8_t* Aq, float* a_scale,
                           int32_t* rowsum, hipStream_t stream);

namespace w4 {

// Argument checks of the fused entry points (everything but the workspace).
int fused_check(int kind, const void* A, int in_dtype, const uint8_t* Wp, const void* scale,
                const uint16_t* bias, void* C, int out_dtype, int M, int N, int K) {
  if (in_dtype != W4_IN_F16 && in_dtype != W4_IN_F32) return W4_ERR_ARG;
  if (out_dtype != W4_OUT_F16 && out_dtype != W4_OUT_F32 && out_dtype != W4_OUT_I32)
    return W4_ERR_ARG;
  const int st = check_common(M, N, K, 16);
  if (st != W4_OK) return st;
  if (M == 0) return W4_OK;
  if (!A || !Wp || !scale || !C) return W4_ERR_NULL;
  if (!aligned(A, 16) || !aligned(Wp, 16) || !out_aligned(C, out_dtype) ||
      (bias && !aligned(bias, 2)) || !aligned(scale, kind == KIND_W4A8 ? 4 : 2))
    return W4_ERR_ALIGN;
  return W4_OK;
}

// The fused call: quantize_a8 into the workspace and the A8 matmul (two
// launches), or one decode kernel that quantizes in its prologue.
int fused_common(int kind, const void* A, int in_dtype, const uint8_t* Wp, const void* scale,
                 const uint16_t* bias, void* C, int out_dtype, int M, int N, int K, void* ws,
                 size_t ws_bytes, hipStream_t stream) {
  const int st = fused_check(kind, A, in_dtype, Wp, scale, bias, C, out_dtype, M, N, K);
  if (st != W4_OK || M == 0) return st;
  const FusedPlan F = fused_plan(kind, M, N, K);
  if (F.ws_bytes) {
    if (!ws || ws_bytes < F.ws_bytes) return W4_ERR_WORKSPACE;
    if (!aligned(ws, 256)) return W4_ERR_ALIGN;
  }
  uint8_t* wsb = reinterpret_cast<uint8_t*>(ws);
  const Geometry g = geometry(kind_layout(kind), N, K);
  const int fq = in_dtype == W4_IN_F16 ? 1 : 2;
  if (!F.fqc) {
    int8_t* Aq = reinterpret_cast<int8_t*>(wsb + F.q_off);
    float* sa = reinterpret_cast<float*>(wsb + F.q_off + align256((size_t)M * K));
    const int q = quantize_a8(A, in_dtype, M, K, Aq, sa, nullptr, stream);
    if (q != W4_OK) return q;
    return a8_common(kind, Aq, sa, Wp, scale, bias, C, out_dtype, M, N, K, wsb, F.q_off, stream);
  }
  MMParams p{};
  p.A = A;
  p.Wt = Wp;
  p.w_scale = kind == KIND_W4A8 ? (const float*)scale : nullptr;
  p.w_scale16 = kind == KIND_W2A8 ? (const uint16_t*)scale : nullptr;
  p.bias = out_dtype == W4_OUT_I32 ? nullptr : bias;
  p.C = C;
  p.out_dtype = out_dtype;
  p.M = M;
  p.N = N;
  p.K = K;
  p.NT = g.NT;
  p.KT = g.KT;
  p.KQ = g.KQ;
  return kind == KIND_W4A8 ? launch_gemv<KIND_W4A8>(F.P, p, ws, stream, fq, F.fqc)
                           : launch_gemv<KIND_W2A8>(F.P, p, ws, stream, fq, F.fqc);
}

}  // namespace w4

extern "C" int w4a8_gemm_fused_act(const void* A, int in_dtype, const uint8_t* Wp,
                                   const float* w_scale, const uint16_t* bias, void* C,
                                   int out_dtype, int M, int N, int K, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream) {
  return fused_common(KIND_W4A8, A, in_dtype, Wp, w_scale, bias, C, out_dtype, M, N, K, workspace,
                      workspace_bytes, stream);
}

extern "C" int w2a8_gemm_fused_act(const void* A, int in_dtype, const uint8_t* Wp,
                                   const uint16_t* w_scale16, const uint16_t* bias, void* C,
                                   int out_dtype, int M, int N, int K, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream) {
  return fused_common(KIND_W2A8, A, in_dtype, Wp, w_scale16, bias, C, out_dtype, M, N, K,
                      workspace, workspace_bytes, stream);
}

extern "C" int w2a16_gemm(const uint16_t* A, const uint8_t* Wp, const uint16_t* w_scale16,
                          const uint16_t* bias, uint16_t* C, int M, int N, int K, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  const int st = check_common(M, N, K, 16);
  if (st != W4_OK) return st;
  if (M == 0) return W4_OK;
  if (!A || !Wp || !w_scale16 || !C) return W4_ERR_NULL;
  if (!aligned(A, 16) || !aligned(Wp, 16) || !aligned(C, 2) || !aligned(w_scale16, 2) ||
      (bias && !aligned(bias, 2)))
    return W4_ERR_ALIGN;
  MMParams p{};
  p.A = A;
  p.Wt = Wp;
  p.w_scale16 = w_scale16;
  p.bias = bias;
  p.C = C;
  p.out_dtype = W4_OUT_F16;
  p.M = M;
  p.N = N;
  p.K = K;
  return run<KIND_W2A16>(p, workspace, workspace_bytes, stream);
}

extern "C" int w8a8_gemm(const int8_t* Aq, const float* a_scale, const uint8_t* Wp,
                         const float* w_scale, const uint16_t* bias, const float* out_scale,
                         void* C, int out_dtype, int M, int N, int K, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  if (out_dtype != W4_OUT_F16 && out_dtype != W4_OUT_F32 && out_dtype != W4_OUT_I32 &&
      out_dtype != W4_OUT_I8)
    return W4_ERR_ARG;
  if (out_dtype == W4_OUT_I8 && bias) return W4_ERR_ARG;
  const int st = check_common(M, N, K, 16);
  if (st != W4_OK) return st;
  if (M == 0) return W4_OK;
  if (!Aq || !a_scale || !Wp || !w_scale || !C || (out_dtype == W4_OUT_I8 && !out_scale))
    return W4_ERR_NULL;
  if (!aligned(Aq, 16) || !aligned(Wp, 16) || !aligned(a_scale, 4) || !aligned(w_scale, 4) ||
      (out_dtype != W4_OUT_I8 && !out_aligned(C, out_dtype)) || (bias && !aligned(bias, 2)) ||
      (out_scale && !aligned(out_scale, 4)))
    return W4_ERR_ALIGN;
  MMParams p{};
  p.A = Aq;
  p.a_scale = a_scale;
  p.Wt = Wp;
  p.w_scale = w_scale;
  p.bias = (out_dtype == W4_OUT_I32 || out_dtype == W4_OUT_I8) ? nullptr : bias;
  p.out_scale = out_scale;
  p.C = C;
  p.out_dtype = out_dtype;
  p.M = M;
  p.N = N;
  p.K = K;
  return run<KIND_W8A8>(p, workspace, workspace_bytes, stream);
}

extern "C" int f8f8_gemm(const uint8_t* Aq, const float* a_scale, const uint8_t* Wp,
                         const float* w_scale, const uint16_t* bias, void* C, int out_dtype, int M,
                         int N, int K, void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
  if (out_dtype != W4_OUT_F16 && out_dtype != W4_OUT_F32) return W4_ERR_ARG;
  const int st = check_common(M, N, K, 16);
  if (st != W4_OK) return st;
  if (M == 0) return W4_OK;
  if (!Aq || !a_scale || !Wp || !w_scale || !C) return W4_ERR_NULL;
  if (!aligned(Aq, 16) || !aligned(Wp, 16) || !aligned(a_scale, 4) || !aligned(w_scale, 4) ||
      !out_aligned(C, out_dtype) || (bias && !aligned(bias, 2)))
    return W4_ERR_ALIGN;
  MMParams p{};
  p.A = Aq;
  p.a_scale = a_scale;
  p.Wt = Wp;
  p.w_scale = w_scale;
  p.bias = out_dtype == W4_OUT_F32 ? nullptr : bias;
  p.C = C;
  p.out_dtype = out_dtype;
  p.M = M;
  p.N = N;
  p.K = K;
  return run<KIND_F8F8>(p, workspace, workspace_bytes, stream);
}

// ---------------------------------------------------------------------------
// plan table: list, name, pin and query the plans a shape may run with
// ---------------------------------------------------------------------------
namespace w4 {

// op code -> kind (the op codes equal the kind codes) and the K multiple
inline int op_check(int op, int M, int N, int K) {
  if (op < KIND_W4A8 || op > KIND_F8F8) return W4_ERR_ARG;
  const int st = check_common(M, N, K, op == KIND_W4A16 ? W4_GROUP_SIZE : 16);
  if (st != W4_OK) return st;
  return M < 1 ? W4_ERR_SHAPE : W4_OK;
}

inline int candidate_name(int kind, const Candidate& c, int M, int N, int K, char* buf,
                          size_t len) {
  int n;
  if (c.path == PATH_GEMM) {
    // block tile: 64 rows per m wave group, 16 columns per n tile
    const int ks = gemm_grid(kind, M, N, K, c.cfg).ksplit;
    n = ks > 1 ? snprintf(buf, len, "gemm:%dx%d,ksplit=%d", 64 * c.cfg.wm, 16 * c.cfg.ntiles, ks)
               : snprintf(buf, len, "gemm:%dx%d", 64 * c.cfg.wm, 16 * c.cfg.ntiles);
  } else if (c.path == PATH_SKINNY) {
    const Plan P = plan_from(kind, M, N, K, c);
    char rows[16] = "";
    if (P.mtb > 1) snprintf(rows, sizeof(rows), ":rows=%d", 16 * P.mtb);
    n = P.ksplit > 1 ? snprintf(buf, len, "skinny%s%sksplit=%d", rows, P.mtb > 1 ? "," : ":",
                                P.ksplit)
                     : snprintf(buf, len, "skinny%s", rows);
  } else {
    const Plan P = plan_from(kind, M, N, K, c);
    n = P.waves != 8 ? snprintf(buf, len, "decode:ksplit=%d,waves=%d", P.ksplit, P.waves)
                     : snprintf(buf, len, "decode:ksplit=%d", P.ksplit);
  }
  return n < 0 || (size_t)n >= len ? W4_ERR_ARG : W4_OK;
}

}  // namespace w4

extern "C" int w4_plan_count(int op, int M, int N, int K) {
  const int st = op_check(op, M, N, K);
  if (st != W4_OK) return st;
  Candidate c[MAX_CANDIDATES];
  return candidates(op, M, N, K, c);
}

extern "C" int w4_plan_name(int op, int M, int N, int K, int index, char* buf, size_t len) {
  const int st = op_check(op, M, N, K);
  if (st != W4_OK) return st;
  if (!buf) return W4_ERR_NULL;
  Candidate c[MAX_CANDIDATES];
  const int n = candidates(op, M, N, K, c);
  if (index < 0 || index >= n || len == 0) return W4_ERR_ARG;
  return candidate_name(op, c[index], M, N, K, buf, len);
}

extern "C" int w4_plan_pin(int op, int M, int N, int K, int index) {
  const int st = op_check(op, M, N, K);
  if (st != W4_OK) return st;
  Candidate c[MAX_CANDIDATES];
  const int n = candidates(op, M, N, K, c);
  if (index < -1 || index >= n) return W4_ERR_ARG;
  std::lock_guard<std::mutex> lock(pin_mutex());
  auto& t = pin_table();
  const ShapeKey key{op, M, N, K};
  if (index < 0) t.erase(key);
  else t[key] = c[index];
  pin_count().store((int)t.size(), std::memory_order_release);
  return W4_OK;
}

extern "C" int w4_plan_current(int op, int M, int N, int K) {
  const int st = op_check(op, M, N, K);
  if (st != W4_OK) return st;
  Candidate c[MAX_CANDIDATES];
  const int n = candidates(op, M, N, K, c);
  const Plan cur = make_plan(op, M, N, K);
  for (int i = 0; i < n; ++i)
    if (same_plan(plan_from(op, M, N, K, c[i]), cur)) return i;
  return W4_ERR_ARG;   // not reached: the built-in choice is always a candidate
}

extern "C" size_t w4_plan_workspace_bytes(int op, int M, int N, int K) {
  if (op_check(op, M, N, K) != W4_OK) return 0;
  return make_plan(op, M, N, K).ws_bytes;
}

extern "C" int w4_plan_reset(void) {
  std::lock_guard<std::mutex> lock(pin_mutex());
  pin_table().clear();
  pin_count().store(0, std::memory_order_release);
  return W4_OK;
}
