// Peak-rate probes for the roofline report (include/s5_peak.h): a streaming
// copy for the HBM rate and a register-only MFMA loop for the matrix-core
// rate. Measurement of the chip only; nothing here is part of the S5 path.
#include <hip/hip_runtime.h>

#include "s5_peak.h"

namespace {

constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;   // 16-byte words in flight per thread

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ __forceinline__ uint4 ld16(const uint4* p) {
  if constexpr (NT) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
  } else {
    return *p;
  }
}
template <bool NT>
__device__ __forceinline__ void st16(uint4* p, const uint4& v) {
  if constexpr (NT) {
    __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4*>(p));
  } else {
    *p = v;
  }
}

// NT: nontemporal (streaming) loads and stores
template <bool NT>
__global__ void __launch_bounds__(kCopyThreads) k_peak_copy(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                            int64_t n) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kCopyThreads;
  int64_t i = static_cast<int64_t>(blockIdx.x) * kCopyThreads + threadIdx.x;
  // whole rounds of kCopyUnroll words per thread, then the remainder
  for (; i + (kCopyUnroll - 1) * stride < n; i += kCopyUnroll * stride) {
    uint4 v[kCopyUnroll];
#pragma unroll
    for (int k = 0; k < kCopyUnroll; ++k) v[k] = ld16<NT>(src + i + k * stride);
#pragma unroll
    for (int k = 0; k < kCopyUnroll; ++k) st16<NT>(dst + i + k * stride, v[k]);
  }
  for (; i < n; i += stride) st16<NT>(dst + i, ld16<NT>(src + i));
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kChains = 8;

__global__ void __launch_bounds__(256) k_peak_mfma(int iters, float* __restrict__ out) {
  // small exact operands (2^-10 and 2^-9): the sums stay far from overflow
  bf16x8 a, b;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    a[k] = static_cast<__bf16>(((threadIdx.x + k) & 1) ? 0.0009765625f : -0.0009765625f);
    b[k] = static_cast<__bf16>(0.001953125f);
  }
  f32x4 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  // four rounds per trip (iters is rounded down to a multiple of four): the
  // accumulators keep their registers across trips
  for (int it = 0; it < iters; it += 4) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < kChains; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  out[static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x] = s;
}

}  // namespace

extern "C" {

int s5_peak_copy(const void* src, void* dst, int64_t bytes, int nontemporal, hipStream_t stream) {
  if (src == nullptr || dst == nullptr || bytes <= 0 || (bytes & 15) != 0) return -1;
  if ((reinterpret_cast<uintptr_t>(src) & 15) != 0 || (reinterpret_cast<uintptr_t>(dst) & 15) != 0) return -1;
  const char* s = static_cast<const char*>(src);
  const char* d = static_cast<const char*>(dst);
  if (s < d + bytes && d < s + bytes) return -1;
  int dev = 0, ncu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu <= 0)
    ncu = 256;
  const int64_t n = bytes / 16;
  int64_t blocks = (n + kCopyThreads - 1) / kCopyThreads;
  if (blocks > 8 * static_cast<int64_t>(ncu)) blocks = 8 * static_cast<int64_t>(ncu);
  if (nontemporal) {
    hipLaunchKernelGGL(k_peak_copy<true>, dim3(static_cast<unsigned>(blocks)), dim3(kCopyThreads), 0, stream,
                       static_cast<const uint4*>(src), static_cast<uint4*>(dst), n);
  } else {
    hipLaunchKernelGGL(k_peak_copy<false>, dim3(static_cast<unsigned>(blocks)), dim3(kCopyThreads), 0, stream,
                       static_cast<const uint4*>(src), static_cast<uint4*>(dst), n);
  }
  return static_cast<int>(hipGetLastError());
}

int s5_peak_mfma_bf16(int blocks, int iters, float* out, hipStream_t stream) {
  if (blocks < 1 || iters < 4 || (iters & 3) != 0 || out == nullptr) return -1;
  hipLaunchKernelGGL(k_peak_mfma, dim3(blocks), dim3(256), 0, stream, iters, out);
  return static_cast<int>(hipGetLastError());
}

}  // extern "C"
