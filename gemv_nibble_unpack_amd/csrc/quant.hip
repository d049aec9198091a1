// Offline weight quantization/packing and per-call activation quantization.
//
// Weight side: INT4 quantization page ("Accelerating LLM inference with CUDA
// Graph and INT4 quantization"), Part 1 step 1, with the INT4 range [-7, 7];
// BitBLAS practical-guide page, "Advanced features 2: weight group
// quantization" (group 128, scales, zeros, zeros_mode original); BitBLAS
// data-type table row INT8 x INT2 for the ternary packing.
// Activation side: INT4 quantization page, Part 1 step 2 (dynamic scale,
// round), per token, range [-127, 127].
//
// Every code-deciding operation is an IEEE float32 division followed by
// round-half-to-even (v_rndne_f32), the same precision in which the codes are
// defined; the library is built without fast-math so '/' is correctly
// rounded.

#include "common.hpp"

namespace w4 {

constexpr int QB = 256;  // threads per block for the row kernels

__device__ __forceinline__ float block_max(float v, float* sh) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) sh[w] = v;
  __syncthreads();
  float r = sh[0];
#pragma unroll
  for (int i = 1; i < QB / 64; ++i) r = fmaxf(r, sh[i]);
  __syncthreads();
  return r;
}

__device__ __forceinline__ int block_sum_i(int v, int* sh) {
  v = wave_sum_i(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) sh[w] = v;
  __syncthreads();
  int r = 0;
#pragma unroll
  for (int i = 0; i < QB / 64; ++i) r += sh[i];
  __syncthreads();
  return r;
}


// --- symmetric per-channel INT4: one block per row n -----------------------
__global__ __launch_bounds__(QB) void k_quant_w4_sym(const float* __restrict__ W, int K,
                                                       uint8_t* __restrict__ Wq,
                                                       float* __restrict__ scales) {
  __shared__ float sh[QB / 64];
  const int n = blockIdx.x;
  const float* row = W + (size_t)n * K;
  float m = 0.f;
  for (int k = threadIdx.x; k < K; k += QB) m = fmaxf(m, fabsf(row[k]));
  m = block_max(m, sh);
  const float s = m / 7.0f;
  if (threadIdx.x == 0) scales[n] = s;
  uint8_t* out = Wq + (size_t)n * (K / 2);
  for (int j = threadIdx.x; j < K / 2; j += QB) {
    const int q0 = sym_code_div(row[2 * j], s, 7.f);
    const int q1 = sym_code_div(row[2 * j + 1], s, 7.f);
    out[j] = (uint8_t)((q0 & 15) | ((q1 & 15) << 4));
  }
}

// --- symmetric per-channel INT8 (the page's /127 formula): one block per row
__global__ __launch_bounds__(QB) void k_quant_w8_sym(const float* __restrict__ W, int K,
                                                       int8_t* __restrict__ Wq,
                                                       float* __restrict__ scales) {
  __shared__ float sh[QB / 64];
  const int n = blockIdx.x;
  const float* row = W + (size_t)n * K;
  float m = 0.f;
  for (int k = threadIdx.x; k < K; k += QB) m = fmaxf(m, fabsf(row[k]));
  m = block_max(m, sh);
  const float s = m / 127.0f;
  if (threadIdx.x == 0) scales[n] = s;
  int8_t* out = Wq + (size_t)n * K;
  for (int k = threadIdx.x; k < K; k += QB) out[k] = (int8_t)sym_code_div(row[k], s, 127.f);
}

// --- asymmetric group-128 uINT4: one wave per (row, group) -----------------
__global__ __launch_bounds__(QB) void k_quant_w4_group(const float* __restrict__ W, int N, int K,
                                                         uint8_t* __restrict__ Wq,
                                                         uint16_t* __restrict__ scales,
                                                         uint8_t* __restrict__ zeros) {
  const int G = K / W4_GROUP_SIZE;
  const size_t gid = (size_t)blockIdx.x * (QB / 64) + (threadIdx.x >> 6);
  if (gid >= (size_t)N * G) return;  // whole wave exits together
  const int lane = threadIdx.x & 63;
  const size_t n = gid / G;
  const int g = (int)(gid % G);
  const float* src = W + n * K + (size_t)g * W4_GROUP_SIZE + 2 * lane;
  const float w0 = src[0], w1 = src[1];
  const float mn = wave_min(fminf(w0, w1));
  const float mx = wave_max(fmaxf(w0, w1));
  const uint16_t s16 = f2h((mx - mn) / 15.0f);
  const float sf = h2f(s16);
  int q0 = 0, q1 = 0, z = 0;
  if (sf > 0.f) {
    const float zf = fminf(fmaxf(rintf(-mn / sf), 0.f), 15.f);
    z = (int)zf;
    q0 = (int)fminf(fmaxf(rintf(w0 / sf) + zf, 0.f), 15.f);
    q1 = (int)fminf(fmaxf(rintf(w1 / sf) + zf, 0.f), 15.f);
  }
  Wq[n * (K / 2) + (size_t)g * (W4_GROUP_SIZE / 2) + lane] = (uint8_t)(q0 | (q1 << 4));
  if (lane == 0) {
    scales[n * G + g] = s16;
    zeros[n * G + g] = (uint8_t)z;
  }
}

// --- ternary packing: one thread per output byte ----------------------------
__global__ __launch_bounds__(QB) void k_pack_w2(const int8_t* __restrict__ codes, size_t nbytes,
                                                  uint8_t* __restrict__ Wq) {
  const size_t i = (size_t)blockIdx.x * QB + threadIdx.x;
  if (i >= nbytes) return;
  const uint32_t c = *reinterpret_cast<const uint32_t*>(codes + 4 * i);
  const uint32_t b = (c & 3u) | (((c >> 8) & 3u) << 2) | (((c >> 16) & 3u) << 4) |
                     (((c >> 24) & 3u) << 6);
  Wq[i] = (uint8_t)b;
}

// --- ternary per-tensor scale: single block, fixed-order float64 sum --------
__device__ uint16_t double_to_half_rne(double x) {
  // x is a finite mean of magnitudes (>= 0). Round once from float64 to the
  // nearest fp16 (ties to even) by scaling to the fp16 quantum of x's binade.
  if (!(x > 0.0)) return 0;
  if (x >= 65520.0) return 0x7C00;
  const int e = ilogb(x);
  const int qexp = e < -14 ? -24 : e - 10;
  const double r = ldexp(rint(ldexp(x, -qexp)), qexp);  // exact fp16 value
  return f2h((float)r);
}

constexpr int TSB = 1024;
__global__ __launch_bounds__(TSB) void k_ternary_scale(const float* __restrict__ src,
                                                         int64_t count,
                                                         uint16_t* __restrict__ out) {
  __shared__ double sh[TSB / 64];
  double acc = 0.0;
  for (int64_t i = threadIdx.x; i < count; i += TSB) acc += (double)fabsf(src[i]);
  acc = wave_sum_d(acc);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    double s = 0.0;
    for (int i = 0; i < TSB / 64; ++i) s += sh[i];
    out[0] = double_to_half_rne(s / (double)count);
  }
}

// --- per-token INT8 activations: one block per row m ------------------------
template <typename T>
__device__ __forceinline__ void load8(const T* p, float (&x)[8]);

template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float (&x)[8]) {
  const u4 v = *reinterpret_cast<const u4*>(p);
  const h8 h = __builtin_bit_cast(h8, v);
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = (float)h[i];
}

template <>
__device__ __forceinline__ void load8<float>(const float* p, float (&x)[8]) {
  const f4 a = *reinterpret_cast<const f4*>(p);
  const f4 b = *reinterpret_cast<const f4*>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[i] = a[i];
    x[4 + i] = b[i];
  }
}

// One block per row m. CPT > 0: the row is read once into registers
// (CPT chunks of 8 elements per thread, K <= 8 * QB * CPT); CPT == 0: two
// passes over the row (the second read hits L2).
template <typename T, int CPT>
__global__ __launch_bounds__(QB) void k_quant_a8(const T* __restrict__ A, int K,
                                                   int8_t* __restrict__ Aq,
                                                   float* __restrict__ a_scale,
                                                   int32_t* __restrict__ rowsum) {
  __shared__ float shf[QB / 64];
  __shared__ int shi[QB / 64];
  const int m = blockIdx.x;
  const T* row = A + (size_t)m * K;
  const int nch = K / 8;
  float mx = 0.f;
  float x[CPT > 0 ? CPT : 1][8];
  if constexpr (CPT > 0) {
    // every chunk load is issued before any is used: unconditional (chunks
    // past the row re-read its last chunk and are zeroed after the loads), as
    // a load inside a branch would be waited for inside it, one chunk after
    // the other
#pragma unroll
    for (int i = 0; i < CPT; ++i) load8<T>(row + 8 * min((int)threadIdx.x + i * QB, nch - 1), x[i]);
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      if ((int)threadIdx.x + i * QB >= nch) {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[i][e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(x[i][e]));
    }
  } else {
    for (int c = threadIdx.x; c < nch; c += QB) {
      float y[8];
      load8<T>(row + 8 * c, y);
#pragma unroll
      for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(y[e]));
    }
  }
  mx = block_max(mx, shf);
  const float s = mx / 127.0f;
  const float rs = s > 0.f ? 1.0f / s : 0.f;
  int sum = 0;
  int8_t* out = Aq + (size_t)m * K;
  auto emit = [&](int c, const float (&y)[8]) {
    uint32_t lo, hi;
    codes8_i8(y, s, rs, lo, hi, sum);
    *reinterpret_cast<u2*>(out + 8 * c) = u2{lo, hi};
  };
  if constexpr (CPT > 0) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = threadIdx.x + i * QB;
      if (c < nch) emit(c, x[i]);
    }
  } else {
    for (int c = threadIdx.x; c < nch; c += QB) {
      float y[8];
      load8<T>(row + 8 * c, y);
      emit(c, y);
    }
  }
  if (threadIdx.x == 0) a_scale[m] = s;
  if (rowsum) {                                      // uniform: a kernel argument
    sum = block_sum_i(sum, shi);
    if (threadIdx.x == 0) rowsum[m] = sum;
  }
}

}  // namespace w4

using namespace w4;

// --- per-row FP8 E4M3 (weights per output channel, activations per token) --
// BitBLAS data-type table, row FP8_E4M3 x FP8_E4M3, in the OCP E4M3 format:
// bias 7, 3 mantissa bits, subnormals below 2^-6 in steps of 2^-9, largest
// finite magnitude 448, no infinities. Scale = max|x| / 448 per row, like the
// INT8 rows' max / 127.
//
// Code of a float32 value: round to nearest, ties to even, sign kept (also for
// zero), magnitude saturated at 448. Normal range: scale the value to [8, 16)
// by a power of two (exact), round to an integer (8 + mantissa; 16 carries
// into the next exponent, which the code arithmetic does by itself).
__device__ __forceinline__ uint32_t e4m3_code(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fminf(fabsf(x), 448.0f);
  uint32_t mag;
  if (a < 0.015625f) {
    mag = (uint32_t)__builtin_rintf(a * 512.0f);           // 0..8 (8 is 2^-6, code 0x08)
  } else {
    const int e = (int)((__float_as_uint(a) >> 23) & 0xFFu) - 127;   // -6 <= e <= 8
    const uint32_t m = (uint32_t)__builtin_rintf(ldexpf(a, 3 - e));  // 8..16
    mag = (uint32_t)(e + 7) * 8u + m - 8u;
  }
  return sign | mag;
}

// One block per row: the row max, then the codes, 8 elements per chunk.
template <typename T>
__global__ __launch_bounds__(QB) void k_quant_f8(const T* __restrict__ X, int K,
                                                  uint8_t* __restrict__ Xq,
                                                  float* __restrict__ scales) {
  __shared__ float sh[QB / 64];
  const int rr = blockIdx.x;
  const T* row = X + (size_t)rr * K;
  float m = 0.f;
  for (int c = threadIdx.x; c < K / 8; c += QB) {
    float x[8];
    load8<T>(row + 8 * c, x);
#pragma unroll
    for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(x[e]));
  }
  m = block_max(m, sh);
  const float s = m / 448.0f;
  if (threadIdx.x == 0) scales[rr] = s;
  uint8_t* out = Xq + (size_t)rr * K;
  for (int c = threadIdx.x; c < K / 8; c += QB) {
    float x[8];
    load8<T>(row + 8 * c, x);
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t q = s > 0.f ? e4m3_code(x[e] / s) : 0u;   // zero row: code 0
      if (e < 4) lo |= q << (8 * e);
      else hi |= q << (8 * (e - 4));
    }
    *reinterpret_cast<u2*>(out + 8 * c) = u2{lo, hi};
  }
}

extern "C" const char* w4_status_string(int status) {
  switch (status) {
    case W4_OK: return "ok";
    case W4_ERR_NULL: return "a required pointer is NULL";
    case W4_ERR_SHAPE: return "a size is out of range or not a required multiple";
    case W4_ERR_ALIGN: return "a pointer is not aligned as required";
    case W4_ERR_ARG: return "an enumerated argument has an unknown value";
    case W4_ERR_WORKSPACE: return "workspace is NULL or too small";
    case W4_ERR_HIP: return "the HIP runtime rejected the launch";
    case W4_ERR_SCRATCH:
      return "the call needs more scratch than the library's static buffer holds "
             "(W4_NOALLOC_SCRATCH_BYTES); use the entry point that takes a workspace";
    default: return "unknown status";
  }
}

extern "C" int quantize_pack_w4(const float* W, int N, int K, int scheme, int group_size,
                                uint8_t* Wq, void* scales, uint8_t* zeros, hipStream_t stream) {
  if (!W || !Wq || !scales) return W4_ERR_NULL;
  if (scheme != W4_SYM_PER_CHANNEL && scheme != W4_ASYM_GROUP) return W4_ERR_ARG;
  if (N < 1 || K < 2 || K % 2 || K > W4_MAX_K) return W4_ERR_SHAPE;
  if (!aligned(W, 16) || !aligned(Wq, 16)) return W4_ERR_ALIGN;
  if (scheme == W4_SYM_PER_CHANNEL) {
    if (group_size != -1) return W4_ERR_ARG;
    if (zeros) return W4_ERR_ARG;
    if (!aligned(scales, 4)) return W4_ERR_ALIGN;
    hipLaunchKernelGGL(k_quant_w4_sym, dim3(N), dim3(QB), 0, stream, W, K, Wq, (float*)scales);
    return launch_status();
  }
  if (group_size != W4_GROUP_SIZE) return W4_ERR_ARG;
  if (!zeros) return W4_ERR_NULL;
  if (K % W4_GROUP_SIZE) return W4_ERR_SHAPE;
  if (!aligned(scales, 2)) return W4_ERR_ALIGN;
  const size_t groups = (size_t)N * (K / W4_GROUP_SIZE);
  const size_t blocks = (groups + QB / 64 - 1) / (QB / 64);
  hipLaunchKernelGGL(k_quant_w4_group, dim3((unsigned)blocks), dim3(QB), 0, stream, W, N, K, Wq,
                     (uint16_t*)scales, zeros);
  return launch_status();
}

extern "C" int quantize_pack_w8(const float* W, int N, int K, int8_t* Wq, float* scales,
                                hipStream_t stream) {
  if (!W || !Wq || !scales) return W4_ERR_NULL;
  if (N < 1 || K < 16 || K % 16 || K > W4_MAX_K) return W4_ERR_SHAPE;
  if (!aligned(W, 16) || !aligned(Wq, 16) || !aligned(scales, 4)) return W4_ERR_ALIGN;
  hipLaunchKernelGGL(k_quant_w8_sym, dim3(N), dim3(QB), 0, stream, W, K, Wq, scales);
  return launch_status();
}

extern "C" int quantize_f8(const void* X, int in_dtype, int rows, int K, uint8_t* Xq,
                           float* scales, hipStream_t stream) {
  if (!X || !Xq || !scales) return W4_ERR_NULL;
  if (in_dtype != W4_IN_F16 && in_dtype != W4_IN_F32) return W4_ERR_ARG;
  if (rows < 1 || K < 16 || K % 16 || K > W4_MAX_K) return W4_ERR_SHAPE;
  if (!aligned(X, 16) || !aligned(Xq, 16) || !aligned(scales, 4)) return W4_ERR_ALIGN;
  if (in_dtype == W4_IN_F16)
    hipLaunchKernelGGL(k_quant_f8<uint16_t>, dim3(rows), dim3(QB), 0, stream,
                       (const uint16_t*)X, K, Xq, scales);
  else
    hipLaunchKernelGGL(k_quant_f8<float>, dim3(rows), dim3(QB), 0, stream, (const float*)X, K,
                       Xq, scales);
  return launch_status();
}

extern "C" int quantize_pack_w2(const int8_t* codes, int N, int K, uint8_t* Wq,
                                hipStream_t stream) {
  if (!codes || !Wq) return W4_ERR_NULL;
  if (N < 1 || K < 4 || K % 4 || K > W4_MAX_K) return W4_ERR_SHAPE;
  if (!aligned(codes, 16) || !aligned(Wq, 16)) return W4_ERR_ALIGN;
  const size_t nbytes = (size_t)N * (K / 4);
  hipLaunchKernelGGL(k_pack_w2, dim3((unsigned)((nbytes + QB - 1) / QB)), dim3(QB), 0, stream,
                     codes, nbytes, Wq);
  return launch_status();
}

extern "C" int ternary_scale_f16(const float* src, int64_t count, uint16_t* scale,
                                 hipStream_t stream) {
  if (!src || !scale) return W4_ERR_NULL;
  if (count < 1) return W4_ERR_SHAPE;
  if (!aligned(src, 4) || !aligned(scale, 2)) return W4_ERR_ALIGN;
  hipLaunchKernelGGL(k_ternary_scale, dim3(1), dim3(TSB), 0, stream, src, count, scale);
  return launch_status();
}

extern "C" int quantize_a8(const void* A, int in_dtype, int M, int K, int8_t* Aq, float* a_scale,
                           int32_t* rowsum, hipStream_t stream) {
  if (!A || !Aq || !a_scale) return W4_ERR_NULL;
  if (in_dtype != W4_IN_F16 && in_dtype != W4_IN_F32) return W4_ERR_ARG;
  if (M < 1 || K < 8 || K % 8 || K > W4_MAX_K) return W4_ERR_SHAPE;
  if (!aligned(A, 16) || !aligned(Aq, 16) || !aligned(a_scale, 4) ||
      (rowsum && !aligned(rowsum, 4)))
    return W4_ERR_ALIGN;
  const int cpt = (K / 8 + QB - 1) / QB;            // 8-element chunks per thread
#define W4_QA8(T, C) \
  hipLaunchKernelGGL((k_quant_a8<T, C>), dim3(M), dim3(QB), 0, stream, (const T*)A, K, Aq, a_scale, rowsum)
  if (in_dtype == W4_IN_F16) {
    if (cpt <= 1) W4_QA8(uint16_t, 1);
    else if (cpt <= 2) W4_QA8(uint16_t, 2);
    else if (cpt <= 4) W4_QA8(uint16_t, 4);
    else W4_QA8(uint16_t, 0);
  } else {
    if (cpt <= 1) W4_QA8(float, 1);
    else if (cpt <= 2) W4_QA8(float, 2);
    else if (cpt <= 4) W4_QA8(float, 4);
    else W4_QA8(float, 0);
  }
#undef W4_QA8
  return launch_status();
}
