// The prefill GEMM's kernel instances and their launch (block shape, output
// type and bias, chosen at run time).

#include "gemm.hpp"

namespace w4 {

int launch_gemm_w4a8(const MMParams& p, GemmCfg c, void* ws, hipStream_t stream) {
  const GemmGrid gg = gemm_grid(KIND_W4A8, p.M, p.N, p.K, c);
  if (c.ntiles == 22 && c.wm == 4) return launch_gemm_t<KIND_W4A8, 22, 4>(p, gg, ws, stream);
  if (c.ntiles == 22) return launch_gemm_t<KIND_W4A8, 22, 2>(p, gg, ws, stream);
  return launch_gemm_t<KIND_W4A8, 16, 2>(p, gg, ws, stream);
}

int launch_gemm_w2a8(const MMParams& p, GemmCfg c, void* ws, hipStream_t stream) {
  const GemmGrid gg = gemm_grid(KIND_W2A8, p.M, p.N, p.K, c);
  return launch_gemm_t<KIND_W2A8, 8, 2>(p, gg, ws, stream);
}

int launch_gemm_w8a8(const MMParams& p, GemmCfg c, void* ws, hipStream_t stream) {
  const GemmGrid gg = gemm_grid(KIND_W8A8, p.M, p.N, p.K, c);
  return launch_gemm_t<KIND_W8A8, 8, 2>(p, gg, ws, stream);
}

// FP8: 128 x 128 blocks over the whole K (no workspace)
int launch_gemm_f8f8(const MMParams& p, GemmCfg c, hipStream_t stream) {
  const GemmGrid gg = gemm_grid(KIND_F8F8, p.M, p.N, p.K, c);
  return launch_gemm_t<KIND_F8F8, 8, 2>(p, gg, nullptr, stream);
}

}  // namespace w4
