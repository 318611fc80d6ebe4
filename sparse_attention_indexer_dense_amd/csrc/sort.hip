// sort.hip - rows of a selection reordered into ranking order.
//
// The selection kernels write each row's keys in ascending index order (the
// order a sparse attention gathers them best). indexer_sort_rows rewrites
// rows of (index, score) pairs in place so that they run in ranking order:
// score descending, equal scores by ascending index, -1 padding (score -inf)
// last. One workgroup per row sorts composite 64-bit keys (order-preserving
// score key, complemented index) with a bitonic network in LDS.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.h"
#include "kernels.h"

namespace dsaidx {

constexpr int kSortThreads = 256;

__global__ __launch_bounds__(kSortThreads) void sort_rows_kernel(int32_t *idx, float *score, int64_t rows, int k,
                                                                 int k2)
{
    extern __shared__ uint64_t key[];  // k2 entries (sized at launch: more rows per CU for short rows)
    const int64_t row = blockIdx.x + (int64_t)blockIdx.y * gridDim.x;
    if (row >= rows)
        return;
    int32_t *ri = idx + row * k;
    float *rs = score + row * k;
    for (int i = threadIdx.x; i < k2; i += kSortThreads) {
        uint64_t v = 0;  // below every real entry and every padding entry
        if (i < k)
            v = ((uint64_t)score_key(rs[i] + 0.0f) << 32) | (uint32_t)~(uint32_t)ri[i];
        key[i] = v;
    }
    __syncthreads();
    // descending bitonic sort of k2 (a power of two) keys
    for (int size = 2; size <= k2; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = threadIdx.x; i < k2; i += kSortThreads) {
                const int o = i ^ stride;
                if (o > i) {
                    const uint64_t a = key[i], b = key[o];
                    const bool desc = (i & size) == 0;
                    if (desc ? (a < b) : (a > b)) {
                        key[i] = b;
                        key[o] = a;
                    }
                }
            }
            __syncthreads();
        }
    }
    for (int i = threadIdx.x; i < k; i += kSortThreads) {
        const uint64_t v = key[i];
        ri[i] = (int32_t)~(uint32_t)v;
        rs[i] = key_score((uint32_t)(v >> 32));
    }
}

hipError_t launch_sort_rows(int32_t *idx, float *score, int64_t rows, int k, hipStream_t stream)
{
    int k2 = 1;
    while (k2 < k)
        k2 <<= 1;
    const int64_t gx = rows < 65535 ? rows : 65535;
    const int64_t gy = (rows + gx - 1) / gx;
    hipLaunchKernelGGL(sort_rows_kernel, dim3((unsigned)gx, (unsigned)gy), dim3(kSortThreads),
                       (size_t)k2 * sizeof(uint64_t), stream, idx, score, rows, k, k2);
    return hipGetLastError();
}

}  // namespace dsaidx
