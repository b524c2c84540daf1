// s3r_length_order kernel: the sequences ordered by descending context
// length (ties by index), the order in which draft-step workgroups take them.
//
// rank(i) = #{j : len[j] > len[i]} + #{j < i : len[j] == len[i]} is a
// permutation of 0..B-1; thread i writes order[rank(i)] = i. Every thread
// compares its length with all B lengths, staged through LDS in tiles
// (O(B^2 / 256) per thread; a few microseconds at the batch sizes here).

#include "common.hpp"
#include "kernels.hpp"

namespace s3r {

constexpr int kOrdThreads = 256;
constexpr int kOrdTile = 1024;

__global__ __launch_bounds__(kOrdThreads) void length_order_kernel(const int* __restrict__ len, int B,
                                                                   int* __restrict__ order) {
  __shared__ int tile[kOrdTile];
  const int i = blockIdx.x * kOrdThreads + threadIdx.x;
  const int li = i < B ? len[i] : 0;
  int rank = 0;
  for (int t0 = 0; t0 < B; t0 += kOrdTile) {
    const int n = min(kOrdTile, B - t0);
    __syncthreads();  // the previous tile is no longer read
    for (int t = threadIdx.x; t < n; t += kOrdThreads) tile[t] = len[t0 + t];
    __syncthreads();
    if (i < B) {
      for (int t = 0; t < n; ++t) {
        const int lj = tile[t];
        rank += (lj > li || (lj == li && t0 + t < i)) ? 1 : 0;
      }
    }
  }
  if (i < B) order[rank] = i;
}

hipError_t launch_length_order(const int* len, int B, int* order, hipStream_t stream) {
  hipLaunchKernelGGL(length_order_kernel, dim3(ceil_div(B, kOrdThreads)), dim3(kOrdThreads), 0, stream, len, B,
                     order);
  return hipGetLastError();
}

}  // namespace s3r
