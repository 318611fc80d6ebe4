// batch.hip - small kernels for batches of requests of different lengths:
// writing the request descriptors into the workspace, and marking the
// candidate rows of guarded groups (groups scored as dense rows instead of
// through a proxy, so that they have no candidate set).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace dsaidx {

__global__ __launch_bounds__(64) void set_desc_kernel(DescChunk ch, ReqDesc *dst)
{
    const int i = threadIdx.x;
    if (i < ch.n)
        dst[ch.first + i] = ch.d[i];
}

// grid (guarded groups of the largest request, B): one row of c entries each
__global__ __launch_bounds__(256) void fill_guarded_kernel(const ReqDesc *req, int64_t L, int64_t q_len, int64_t g,
                                                           int64_t m0, int64_t c, int32_t *cand)
{
    const int64_t m = blockIdx.x;
    const Req rq = request_of(req, blockIdx.y, L, q_len, g, m0);
    if (m >= rq.m0 || m >= rq.G)
        return;
    int32_t *row = cand + (rq.g_off + m) * c;
    for (int64_t i = threadIdx.x; i < c; i += blockDim.x)
        row[i] = -1;
}

hipError_t launch_set_desc(const DescChunk &ch, ReqDesc *dst, hipStream_t stream)
{
    hipLaunchKernelGGL(set_desc_kernel, dim3(1), dim3(64), 0, stream, ch, dst);
    return hipGetLastError();
}

hipError_t launch_fill_guarded(const ReqDesc *req, int B, int64_t L, int64_t q_len, int64_t g, int64_t m0,
                               int64_t gmax, int64_t c, int32_t *cand, hipStream_t stream)
{
    hipLaunchKernelGGL(fill_guarded_kernel, dim3((unsigned)gmax, (unsigned)B), dim3(256), 0, stream, req, L, q_len,
                       g, m0, c, cand);
    return hipGetLastError();
}

}  // namespace dsaidx
