// w4a8_gemm_fused_act without a workspace argument, for callers that cannot
// allocate device memory (code under graph capture, tight serving loops,
// harnesses that forbid allocation). Its scratch -- split-K arrival counters
// and partial sums, and the int8 rows of the two-launch form -- is a static
// device array of W4_NOALLOC_SCRATCH_BYTES; each GPU the library runs on
// holds its own copy until the process ends. In host code the array's name
// only stands for it: the device address of a GPU's copy comes from
// hipGetSymbolAddress, taken once per device with that device current, and
// only that address is handed to kernels.

#include <mutex>

#include "common.hpp"

static __device__ __align__(256) uint8_t scratch[W4_NOALLOC_SCRATCH_BYTES];

namespace w4 {

// the fused call and its argument checks (matmul.hip)
int fused_check(int kind, const void* A, int in_dtype, const uint8_t* Wp, const void* scale,
                const uint16_t* bias, void* C, int out_dtype, int M, int N, int K);
int fused_common(int kind, const void* A, int in_dtype, const uint8_t* Wp, const void* scale,
                 const uint16_t* bias, void* C, int out_dtype, int M, int N, int K, void* ws,
                 size_t ws_bytes, hipStream_t stream);

constexpr int KIND_W4A8_OP = W4_OP_W4A8;     // the op codes equal the kernel kinds
constexpr int SCRATCH_DEVICES = 64;

struct ScratchSlot {
  std::once_flag once;
  void* ptr = nullptr;     // this device's copy of `scratch`
  int status = W4_ERR_HIP;
};

inline ScratchSlot* scratch_slots() {
  static ScratchSlot slots[SCRATCH_DEVICES];
  return slots;
}

// zero `n` 32-bit words (a kernel, not a memset, so that a first call made
// under graph capture records nothing but kernels)
__global__ void k_zero_words(uint32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// The current device's scratch address, set up on the first call on that
// device: the symbol's address, then its counter area cleared on `stream`
// (the array starts zeroed when the code object loads, and every call leaves
// the counters zero again; the clear makes the first call independent of
// both).
inline int scratch_ptr(hipStream_t stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= SCRATCH_DEVICES) return W4_ERR_HIP;
  ScratchSlot& slot = scratch_slots()[dev];
  std::call_once(slot.once, [&] {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return;
    const int words = (int)(WS_COUNTERS / sizeof(uint32_t));
    hipLaunchKernelGGL(k_zero_words, dim3(ceil_div(words, 256)), dim3(256), 0, stream,
                       reinterpret_cast<uint32_t*>(p), words);
    if (hipGetLastError() != hipSuccess) return;
    slot.ptr = p;
    slot.status = W4_OK;
  });
  *out = slot.ptr;
  return slot.status;
}

}  // namespace w4

using namespace w4;

extern "C" int w4a8_gemm_fused_act_noalloc(const void* A, int in_dtype, const uint8_t* Wp,
                                           const float* w_scale, const uint16_t* bias, void* C,
                                           int out_dtype, int M, int N, int K,
                                           hipStream_t stream) {
  const int st = fused_check(KIND_W4A8_OP, A, in_dtype, Wp, w_scale, bias, C, out_dtype, M, N, K);
  if (st != W4_OK || M == 0) return st;
  const size_t need = w4_fused_act_workspace_bytes(W4_LAYOUT_W4A8, M, N, K);
  if (need > (size_t)W4_NOALLOC_SCRATCH_BYTES) return W4_ERR_SCRATCH;
  void* ws = nullptr;
  if (need) {
    const int ss = scratch_ptr(stream, &ws);
    if (ss != W4_OK) return ss;
  }
  return fused_common(KIND_W4A8_OP, A, in_dtype, Wp, w_scale, bias, C, out_dtype, M, N, K, ws,
                      need ? (size_t)W4_NOALLOC_SCRATCH_BYTES : 0, stream);
}
