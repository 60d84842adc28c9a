// Measured peaks of the MI355X the path runs on, for the benchmark's
// roofline fractions: a plain device copy (the HBM bandwidth a streaming
// kernel can reach) and a loop of the FP8 matrix instruction the indexer and
// the attention use (the MFMA rate a kernel can reach).  Built as its own
// library (libcsa_peak.so); nothing on the CSA path calls it.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// Grid-stride copy with 16-byte loads, four in flight per thread.
__global__ __launch_bounds__(256) void copy_kernel(const v4i* __restrict__ src, v4i* __restrict__ dst, size_t n16) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const v4i a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    dst[i] = a;
    dst[i + stride] = b;
    dst[i + 2 * stride] = c;
    dst[i + 3 * stride] = d;
  }
  for (; i < n16; i += stride) dst[i] = src[i];
}

// Every wave issues `iters` rounds of kChains independent
// v_mfma_scale_f32_16x16x128_f8f6f4 (FP8 E4M3 operands, unit scales):
// 2 * 16 * 16 * 128 FLOPs each.  Operands come from the thread id, so
// nothing folds; each lane writes its accumulator sum, so nothing is dropped.
constexpr int kChains = 8;
__global__ __launch_bounds__(256) void mfma_fp8_kernel(float* __restrict__ out, int iters) {
  const int tid = blockIdx.x * blockDim.x + threadIdx.x;
  v8i a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = (int)(0x38383838u ^ (uint32_t)(tid * 2654435761u + j));
    b[j] = (int)(0x30303030u ^ (uint32_t)(tid * 40503u + 7 * j));
  }
  // keep the exponent bits small: no NaN/Inf codes in the operands
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] &= 0x3f3f3f3f;
    b[j] &= 0x3f3f3f3f;
  }
  v4f acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = (v4f){0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[c], 0, 0, 0, 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < kChains; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  out[tid] = s;
}

}  // namespace

extern "C" {

// Copies `bytes` (a multiple of 16, both pointers 16-byte aligned) from src
// to dst on `stream` with `blocks` workgroups of 256 threads.  Returns 0, or
// -1 for bad arguments, -3 if the launch failed.
int csa_peak_copy(const void* src, void* dst, size_t bytes, int blocks, void* stream) {
  if (!src || !dst || bytes % 16 || blocks < 1 || ((uintptr_t)src & 15) || ((uintptr_t)dst & 15)) return -1;
  hipLaunchKernelGGL(copy_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, static_cast<const v4i*>(src),
                     static_cast<v4i*>(dst), bytes / 16);
  return hipPeekAtLastError() == hipSuccess ? 0 : -3;
}

// FP8 MFMA loop: `blocks` workgroups of 256 threads, `iters` rounds each;
// out receives blocks * 256 floats.  FLOPs = blocks * 4 waves * iters *
// csa_peak_mfma_chains() * 65536.
int csa_peak_mfma_fp8(float* out, int iters, int blocks, void* stream) {
  if (!out || iters < 1 || blocks < 1) return -1;
  hipLaunchKernelGGL(mfma_fp8_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, out, iters);
  return hipPeekAtLastError() == hipSuccess ? 0 : -3;
}

int csa_peak_mfma_chains(void) { return kChains; }

}  // extern "C"
