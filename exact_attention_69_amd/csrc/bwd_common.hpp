// Backward preprocessing shared by the bf16 and fp32 paths.
#pragma once

#include "device_common.hpp"

namespace exattn {

// D_i = sum_k dO_ik * O_ik in fp32 (the row term of dS = P * (dP - D) that
// the chain rule of the softmax produces), stored negated: the bf16 gradient
// kernels start the accumulator of the dP product at -D, so the product
// delivers dP - D and dS takes one multiply per element.  Also LSE_i *
// log2(e), the base-2 form of the log-sum-exp that the gradient kernels
// subtract from their base-2 scores.  Each thread reduces 8 contiguous elements; the D/8 threads
// of a row combine their partial sums with xor shuffles.  rows = B*H*n.
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_rowdot_kernel(const T* __restrict__ O, const T* __restrict__ dO,
                                                         const float* __restrict__ lse, float* __restrict__ delta,
                                                         float* __restrict__ lse2, long rows) {
  constexpr int TPR = D / 8;  // threads per row
  const long gid = (long)blockIdx.x * 256 + threadIdx.x;
  const long row = gid / TPR;
  const int part = (int)(gid - row * TPR);
  float acc = 0.0f;
  if (row < rows) {
    const T* o = O + row * D + 8 * part;
    const T* g = dO + row * D + 8 * part;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc += (float)o[i] * (float)g[i];
  }
#pragma unroll
  for (int s = TPR / 2; s >= 1; s >>= 1) acc += __shfl_xor(acc, s, 64);
  if (row < rows && part == 0) {
    delta[row] = -acc;
    lse2[row] = lse[row] * kLog2e;
  }
}

template <typename T>
hipError_t launch_rowdot(const T* O, const T* dO, const float* lse, float* delta, float* lse2, long rows, int d,
                         hipStream_t stream) {
  const long threads = rows * (d / 8);
  const unsigned blocks = (unsigned)((threads + 255) / 256);
  switch (d) {
    case 64:
      hipLaunchKernelGGL((bwd_rowdot_kernel<T, 64>), dim3(blocks), dim3(256), 0, stream, O, dO, lse, delta, lse2, rows);
      break;
    case 128:
      hipLaunchKernelGGL((bwd_rowdot_kernel<T, 128>), dim3(blocks), dim3(256), 0, stream, O, dO, lse, delta, lse2,
                         rows);
      break;
    case 256:
      hipLaunchKernelGGL((bwd_rowdot_kernel<T, 256>), dim3(blocks), dim3(256), 0, stream, O, dO, lse, delta, lse2,
                         rows);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace exattn
