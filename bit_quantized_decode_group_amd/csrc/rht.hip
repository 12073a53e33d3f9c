// rht.hip -- input randomised Hadamard transform ahead of an affine-4
// projection (uzu page, section "내부 동작 1", linear row: an input-side
// random Hadamard transform spreads the quantisation error; its Metal kernel
// list names a hadamard_transform).  For each row m and each block of `had`
// consecutive k (had a power of two dividing K):
//   xr = (1/sqrt(had)) H_had diag(s) x,   H[i][j] = (-1)^popcount(i & j),
// with s[k] = -1 where signs[k] < 0, else +1.  The result is written as two
// bf16 planes, hi = bf16(xr) and lo = bf16(xr - hi), so that the projection
// (QG_MODE_PLANES) multiplies the weights by hi + lo, which carries 16
// significant bits of the fp32 transform.
//
// One workgroup per (row, block): the signed values are loaded into LDS in
// fp32, log2(had) butterfly passes (a, b) -> (a + b, a - b) compute H . v in
// natural (Sylvester) order, then the scale and the split.
#include "common.h"

namespace qg {

constexpr int kRhtThreads = 256;

__global__ void __launch_bounds__(kRhtThreads) k_rht(const uint16_t* __restrict__ x, const int8_t* __restrict__ signs,
                                                     int had, int K, uint16_t* __restrict__ hi,
                                                     uint16_t* __restrict__ lo) {
  __shared__ float v[kRhtMax];
  const int nblk = K / had;
  const int m = blockIdx.x / nblk, b = blockIdx.x % nblk;
  const size_t base = (size_t)m * K + (size_t)b * had;
  for (int i = threadIdx.x; i < had; i += blockDim.x) {
    const float xv = bf16_bits_to_f32(x[base + i]);
    v[i] = signs[(size_t)b * had + i] < 0 ? -xv : xv;
  }
  __syncthreads();
  for (int len = 1; len < had; len <<= 1) {
    for (int t = threadIdx.x; t < had / 2; t += blockDim.x) {
      const int i = ((t & ~(len - 1)) << 1) | (t & (len - 1));  // pair (i, i + len), bit `len` of i clear
      const float a = v[i], c = v[i + len];
      v[i] = a + c;
      v[i + len] = a - c;
    }
    __syncthreads();
  }
  const float scale = 1.0f / sqrtf((float)had);
  for (int i = threadIdx.x; i < had; i += blockDim.x) {
    const float r = v[i] * scale;
    const uint16_t h = f32_to_bf16_bits(r);
    hi[base + i] = h;
    lo[base + i] = f32_to_bf16_bits(r - bf16_bits_to_f32(h));
  }
}

}  // namespace qg

int qg_launch_rht(const uint16_t* x, const int8_t* signs, int had, int M, int K, uint16_t* hi, uint16_t* lo,
                  hipStream_t st) {
  const unsigned grid = (unsigned)((size_t)M * (K / had));
  hipLaunchKernelGGL(qg::k_rht, dim3(grid), dim3(qg::kRhtThreads), 0, st, x, signs, had, K, hi, lo);
  return (int)hipGetLastError();
}
