// chunks.hip - the key-axis coarse stage: chunk partitions of the keys,
// mean-key summaries, the chunk limit of every query group, and the expansion
// of selected chunks into candidate key lists for Refine.
//
// SCALE paper ("Not All Tokens Deserve Equal Resolution: Score-Adaptive
// Indexing for Sparse Attention in Long-Context LLMs"), abstract: contiguous
// key regions are represented by their mean key, candidates are chosen among
// the summaries and refined with the token-level indexer; fixed blocks are the
// baseline and SCALE re-partitions the keys, splitting high-dispersion regions
// and merging homogeneous neighbours under the same number of chunks.
//
// A partition is given by the chunk ends cend[B][nc] (exclusive, ascending,
// the last one = L). All kernels here are bandwidth- or latency-bound and
// small next to the scans: they touch every key once (summaries, dispersion)
// or only chunk-level data.
#include <hip/hip_bf16.h>
#include <hip/hip_runtime.h>

#include "device.h"
#include "kernels.h"

namespace dsaidx {

// ------------------------------------------------------------ fixed blocks
__global__ void chunk_fixed_kernel(int B, int64_t L, int64_t block, int64_t nc, int32_t *cend)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)B * nc)
        return;
    const int64_t e = (i % nc + 1) * block;
    cend[i] = (int32_t)(e < L ? e : L);
}

// ---------------------------------------------------------------- summaries
// Mean key of chunks [first, nc) of every request: per dimension an fp32 sum
// over the chunk's keys in index order, an IEEE fp32 division by the number of
// keys, bf16 round-to-nearest-even. A thread owns 8 dimensions of one chunk
// (one 16-byte load per key); the D/8 threads of a chunk read whole key rows.
template <int D>
__global__ __launch_bounds__(256) void chunk_means_kernel(const uint16_t *K, int64_t L, const int32_t *cend,
                                                          int64_t nc, int64_t first, uint16_t *Kbar)
{
    constexpr int TPC = D / 8;         // threads per chunk
    constexpr int CPB = 256 / TPC;     // chunks per workgroup
    const int bi = blockIdx.y;
    const int64_t ch = first + (int64_t)blockIdx.x * CPB + threadIdx.x / TPC;
    if (ch >= nc)
        return;
    const int x = (threadIdx.x % TPC) * 8;
    const int32_t *ce = cend + (int64_t)bi * nc;
    const int64_t a = ch == 0 ? 0 : ce[ch - 1];
    const int64_t e = ce[ch];
    const uint16_t *Kb = K + (int64_t)bi * L * D;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    int64_t s = a;
    // four rows in flight, added in index order
    for (; s + 4 <= e; s += 4) {
        u32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
            v[u] = *reinterpret_cast<const u32x4 *>(Kb + (s + u) * D + x);
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc[2 * q] += __uint_as_float(v[u][q] << 16);
                acc[2 * q + 1] += __uint_as_float(v[u][q] & 0xFFFF0000u);
            }
    }
    for (; s < e; ++s) {
        const u32x4 v = *reinterpret_cast<const u32x4 *>(Kb + s * D + x);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            acc[2 * q] += __uint_as_float(v[q] << 16);
            acc[2 * q + 1] += __uint_as_float(v[q] & 0xFFFF0000u);
        }
    }
    const float n = (float)(e - a);
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t lo = __bfloat16_as_ushort(__float2bfloat16(__fdiv_rn(acc[2 * q], n)));
        const uint32_t hi = __bfloat16_as_ushort(__float2bfloat16(__fdiv_rn(acc[2 * q + 1], n)));
        o[q] = lo | (hi << 16);
    }
    *reinterpret_cast<u32x4 *>(Kbar + ((int64_t)bi * nc + ch) * D + x) = o;
}

// ------------------------------------------------------------ group limits
// Last chunk complete at the group's last position t_last (cend <= t_last + 1),
// -1 if none: the coarse scan of the group covers chunks 0..glim.
__global__ void chunk_limits_kernel(int B, int64_t L, int64_t q_len, int64_t g, const int32_t *cend, int64_t nc,
                                    int32_t *glim)
{
    const int64_t G = (q_len + g - 1) / g;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)B * G)
        return;
    const int64_t bi = i / G, m = i % G;
    const int64_t r1 = ((m + 1) * g < q_len) ? (m + 1) * g : q_len;
    const int64_t lim = L - q_len + r1;  // t_last + 1
    const int32_t *ce = cend + bi * nc;
    int64_t lo = 0, hi = nc;  // first chunk with cend > lim
    while (lo < hi) {
        const int64_t mid = (lo + hi) / 2;
        if (ce[mid] <= lim)
            lo = mid + 1;
        else
            hi = mid;
    }
    glim[i] = (int32_t)(lo - 1);
}

// --------------------------------------------------------------- expansion
// Candidate list of one group: the keys of its selected chunks (ascending,
// -1 after the last), then the keys after its last complete chunk up to
// t_last, then -1 up to cw; cand_n = the number of keys written. One
// workgroup per group; chunks go in tiles of 256, each tile's key offsets
// from a workgroup prefix sum.
constexpr int kExpandThreads = 256;

__global__ __launch_bounds__(kExpandThreads) void chunk_expand_kernel(ChunkExpandParams p)
{
    __shared__ int32_t off[kExpandThreads + 1];
    __shared__ int32_t cst[kExpandThreads];
    __shared__ int32_t wsum[kExpandThreads / kWave];
    const int64_t grp = blockIdx.x;  // bi * G + m
    const int64_t G = (p.q_len + p.g - 1) / p.g;
    const int64_t bi = grp / G, m = grp % G;
    const int64_t r1 = ((m + 1) * p.g < p.q_len) ? (m + 1) * p.g : p.q_len;
    const int64_t t_last = p.L - p.q_len + r1 - 1;
    const int32_t *ce = p.cend + bi * p.nc;
    const int32_t *sel = p.chunks + grp * p.nsel;
    int32_t *out = p.cand + grp * p.cw;
    const int tid = threadIdx.x;
    int64_t base = 0;
    for (int t0 = 0; t0 < p.nsel; t0 += kExpandThreads) {
        const int j = t0 + tid;
        const int32_t b = j < p.nsel ? sel[j] : -1;
        const int32_t a = b > 0 ? ce[b - 1] : 0;
        const int32_t n = b >= 0 ? ce[b] - a : 0;
        // inclusive prefix sum of n over the tile
        int32_t x = n;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const int32_t y = __shfl_up(x, d, kWave);
            if ((tid % kWave) >= d)
                x += y;
        }
        if (tid % kWave == kWave - 1)
            wsum[tid / kWave] = x;
        __syncthreads();
        int32_t before = 0;
        for (int w = 0; w < tid / kWave; ++w)
            before += wsum[w];
        off[tid + 1] = before + x;
        cst[tid] = a;
        if (tid == 0)
            off[0] = 0;
        __syncthreads();
        const int32_t total = off[kExpandThreads];
        for (int32_t i = tid; i < total; i += kExpandThreads) {
            // chunk of key slot i: the last c with off[c] <= i
            int lo = 0, hi = kExpandThreads - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) / 2;
                if (off[mid] <= i)
                    lo = mid;
                else
                    hi = mid - 1;
            }
            const int64_t slot = base + i;
            if (slot < p.cw)
                out[slot] = cst[lo] + (i - off[lo]);
        }
        base += total;
        __syncthreads();
    }
    const int32_t gl = p.glim[grp];
    const int64_t tail0 = gl >= 0 ? ce[gl] : 0;
    const int64_t ntail = t_last + 1 - tail0;
    for (int64_t i = tid; i < ntail; i += kExpandThreads) {
        const int64_t slot = base + i;
        if (slot < p.cw)
            out[slot] = (int32_t)(tail0 + i);
    }
    base += ntail > 0 ? ntail : 0;
    const int64_t nv = base < p.cw ? base : p.cw;
    for (int64_t i = nv + tid; i < p.cw; i += kExpandThreads)
        out[i] = -1;
    if (tid == 0)
        p.cand_n[grp] = (int32_t)nv;
}

// ------------------------------------------------------- adaptive chunking
// Dispersion of a range of keys, sum_e (sum_s k_se^2 - (sum_s k_se)^2 / n),
// evaluated exactly as the plain definition orders it: per dimension the two
// sums run over the keys in index order (one multiply and one add per term,
// no fused multiply-add), then the per-dimension terms are added in
// dimension order. The split/merge decisions compare such values, so every
// implementation of the partition must take the same steps to make the same
// decisions.
struct Acc2 {
    double s1, s2;
};

__device__ __forceinline__ void acc_add(Acc2 &a, double x)
{
#pragma clang fp contract(off)
    a.s1 = a.s1 + x;
    const double sq = x * x;
    a.s2 = a.s2 + sq;
}

__device__ __forceinline__ double acc_term(const Acc2 &a, double n)
{
#pragma clang fp contract(off)
    const double m = a.s1 * a.s1;
    const double q = m / n;
    return a.s2 - q;
}

// One workgroup per aligned pair of full blocks (or the last full block when
// their count is odd), one thread per dimension: dispersions of the pair, its
// two blocks and their four halves; split gains of the blocks and the merge
// loss of the pair.
template <int D>
__global__ __launch_bounds__(D) void chunk_disp_kernel(ChunkAdaptParams p)
{
    __shared__ double terms[7][D];
    const int64_t j = blockIdx.x;
    const int bi = blockIdx.y;
    const int e = threadIdx.x;
    const int64_t blk = p.block, h = p.block / 2;
    const bool pair = j < p.npair;
    const int64_t a = (pair ? 2 * j : 2 * p.npair) * blk;
    const int64_t len = pair ? 2 * blk : blk;
    const uint16_t *Kb = p.K + (int64_t)bi * p.L * D;
    // ranges: 0 pair, 1..2 blocks, 3..6 halves (of block 0, then block 1)
    Acc2 r[7];
#pragma unroll
    for (int x = 0; x < 7; ++x)
        r[x] = Acc2{0.0, 0.0};
    for (int64_t s = 0; s < len; ++s) {
        const double x = (double)__uint_as_float((uint32_t)Kb[(a + s) * D + e] << 16);
        if (pair)
            acc_add(r[0], x);
        const int b = (int)(s / blk);
        const int q = (int)(s / h);
        if (b == 0)
            acc_add(r[1], x);
        else
            acc_add(r[2], x);
        switch (q) {
        case 0: acc_add(r[3], x); break;
        case 1: acc_add(r[4], x); break;
        case 2: acc_add(r[5], x); break;
        default: acc_add(r[6], x); break;
        }
    }
    terms[0][e] = pair ? acc_term(r[0], (double)(2 * blk)) : 0.0;
    terms[1][e] = acc_term(r[1], (double)blk);
    terms[2][e] = pair ? acc_term(r[2], (double)blk) : 0.0;
#pragma unroll
    for (int x = 3; x < 7; ++x)
        terms[x][e] = (x < 5 || pair) ? acc_term(r[x], (double)h) : 0.0;
    __syncthreads();
    if (e == 0) {
#pragma clang fp contract(off)
        double disp[7];
        for (int x = 0; x < 7; ++x) {
            double t = 0.0;
            for (int d = 0; d < D; ++d)
                t = t + terms[x][d];
            disp[x] = t;
        }
        double *gain = p.gain + (int64_t)bi * p.nfull;
        const int64_t b0 = pair ? 2 * j : 2 * p.npair;
        gain[b0] = (disp[1] - disp[3]) - disp[4];
        if (pair) {
            gain[b0 + 1] = (disp[2] - disp[5]) - disp[6];
            p.loss[(int64_t)bi * p.npair + j] = (disp[0] - disp[1]) - disp[2];
        }
    }
}

// One workgroup per request: sort the split gains (highest first) and merge
// losses (lowest first), ties to the lower number; the greedy pairing of
// splits and merges while the gain exceeds the loss (passing over a split
// whose pair is merged and a merge that holds a split block or the split
// candidate); then the chunk ends in key order. Up to kAdaptBlocksLds blocks
// the sort runs in LDS, beyond that on the workspace (the same steps through
// generic pointers); the split and merge flags are LDS bitmaps either way.
constexpr int kAdaptThreads = 1024;

struct RankLds {
    double gk[kAdaptBlocksLds];
    int32_t gi[kAdaptBlocksLds];
    double lk[kAdaptBlocksLds / 2];
    int32_t li[kAdaptBlocksLds / 2];
    uint32_t split[kAdaptBlocksMax / 32];
    uint32_t merged[kAdaptBlocksMax / 64];
    int32_t wsum[kAdaptThreads / kWave];
};

__device__ __forceinline__ bool bit_of(const uint32_t *b, int i) { return (b[i >> 5] >> (i & 31)) & 1u; }

// bitonic sort of n2 (a power of two) entries; `before(x, y)` is a strict
// total order; the arrays are in LDS or in global memory written only by this
// workgroup (a barrier separates the passes)
template <typename Before>
__device__ __forceinline__ void bitonic(double *k, int32_t *ix, int n2, Before before)
{
    for (int size = 2; size <= n2; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = threadIdx.x; i < n2; i += kAdaptThreads) {
                const int o = i ^ stride;
                if (o > i) {
                    const bool up = (i & size) == 0;
                    const bool sw = up ? before(k[o], ix[o], k[i], ix[i]) : before(k[i], ix[i], k[o], ix[o]);
                    if (sw) {
                        const double tk = k[i];
                        k[i] = k[o];
                        k[o] = tk;
                        const int32_t ti = ix[i];
                        ix[i] = ix[o];
                        ix[o] = ti;
                    }
                }
            }
            __syncthreads();
        }
    }
}

__global__ __launch_bounds__(kAdaptThreads) void chunk_greedy_kernel(ChunkAdaptParams p)
{
    __shared__ RankLds sm;
    const int bi = blockIdx.x;
    const int tid = threadIdx.x;
    const int nfull = (int)p.nfull, npair = (int)p.npair, n = (int)p.n;
    const int g2 = (int)p.g2, p2 = (int)p.p2;
    const bool lds = n <= kAdaptBlocksLds;
    double *gk = lds ? sm.gk : p.gk + (int64_t)bi * g2;
    int32_t *gi = lds ? sm.gi : p.gi + (int64_t)bi * g2;
    double *lk = lds ? sm.lk : p.lk + (int64_t)bi * p2;
    int32_t *li = lds ? sm.li : p.li + (int64_t)bi * p2;
    const double *gain = p.gain + (int64_t)bi * p.nfull;
    const double *loss = p.loss + (int64_t)bi * p.npair;
    for (int i = tid; i < g2; i += kAdaptThreads) {
        gk[i] = i < nfull ? gain[i] : -__builtin_inf();
        gi[i] = i < nfull ? i : 0x7FFFFFFF;
    }
    for (int i = tid; i < p2; i += kAdaptThreads) {
        lk[i] = i < npair ? loss[i] : __builtin_inf();
        li[i] = i < npair ? i : 0x7FFFFFFF;
    }
    for (int i = tid; i < (n + 31) / 32; i += kAdaptThreads)
        sm.split[i] = 0u;
    for (int i = tid; i < (npair + 31) / 32; i += kAdaptThreads)
        sm.merged[i] = 0u;
    __syncthreads();
    bitonic(gk, gi, g2, [](double ka, int32_t ia, double kb, int32_t ib) {
        return ka > kb || (ka == kb && ia < ib);
    });
    bitonic(lk, li, p2, [](double ka, int32_t ia, double kb, int32_t ib) {
        return ka < kb || (ka == kb && ia < ib);
    });
    if (tid == 0) {
        int ia = 0, ib = 0;
        for (;;) {
            while (ia < nfull && gi[ia] / 2 < npair && bit_of(sm.merged, gi[ia] / 2))
                ++ia;
            while (ib < npair) {
                const int jj = li[ib];
                const bool conflict = bit_of(sm.split, 2 * jj) || bit_of(sm.split, 2 * jj + 1) ||
                                      (ia < nfull && gi[ia] / 2 == jj);
                if (!conflict)
                    break;
                ++ib;
            }
            if (ia >= nfull || ib >= npair || !(gk[ia] > lk[ib]))
                break;
            const int sb = gi[ia], mj = li[ib];
            sm.split[sb >> 5] |= 1u << (sb & 31);
            sm.merged[mj >> 5] |= 1u << (mj & 31);
            ++ia;
            ++ib;
        }
    }
    __syncthreads();
    // chunks contributed by each block (a merged pair counts on its first
    // block); thread t takes the blocks [t R, (t + 1) R): their count, an
    // exclusive scan over the threads, then their chunk ends
    auto chunks_of = [&](int b) {
        const bool in_merged = b / 2 < npair && bit_of(sm.merged, b / 2);
        return in_merged ? (b % 2 == 0 ? 1 : 0) : (bit_of(sm.split, b) ? 2 : 1);
    };
    const int R = (n + kAdaptThreads - 1) / kAdaptThreads;
    const int b0 = tid * R;
    const int b1 = (b0 + R < n) ? b0 + R : n;
    int tot = 0;
    for (int b = b0; b < b1; ++b)
        tot += chunks_of(b);
    int x = tot;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int y = __shfl_up(x, d, kWave);
        if ((tid % kWave) >= d)
            x += y;
    }
    if (tid % kWave == kWave - 1)
        sm.wsum[tid / kWave] = x;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < tid / kWave; ++w)
        before += sm.wsum[w];
    int pos = before + x - tot;
    int32_t *ce = p.cend + (int64_t)bi * n;
    const int64_t blk = p.block, h = p.block / 2;
    for (int b = b0; b < b1; ++b) {
        const int cnt = chunks_of(b);
        if (cnt == 0)
            continue;
        const int64_t a = (int64_t)b * blk;
        const bool in_merged = b / 2 < npair && bit_of(sm.merged, b / 2);
        if (in_merged) {
            ce[pos] = (int32_t)(a + 2 * blk);
        } else if (bit_of(sm.split, b)) {
            ce[pos] = (int32_t)(a + h);
            ce[pos + 1] = (int32_t)(a + blk);
        } else {
            ce[pos] = (int32_t)(a + blk < p.L ? a + blk : p.L);
        }
        pos += cnt;
    }
}

// ------------------------------------------------------------- launchers
hipError_t launch_chunk_fixed(int B, int64_t L, int64_t block, int64_t nc, int32_t *cend, hipStream_t stream)
{
    const int64_t n = (int64_t)B * nc;
    hipLaunchKernelGGL(chunk_fixed_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, B, L, block, nc,
                       cend);
    return hipGetLastError();
}

hipError_t launch_chunk_means(int D, const uint16_t *K, int B, int64_t L, const int32_t *cend, int64_t nc,
                              int64_t first, uint16_t *Kbar, hipStream_t stream)
{
    const int64_t todo = nc - first;
    if (D == 128) {
        constexpr int CPB = 256 / (128 / 8);
        hipLaunchKernelGGL(chunk_means_kernel<128>, dim3((unsigned)((todo + CPB - 1) / CPB), (unsigned)B), dim3(256),
                           0, stream, K, L, cend, nc, first, Kbar);
    } else if (D == 32) {
        constexpr int CPB = 256 / (32 / 8);
        hipLaunchKernelGGL(chunk_means_kernel<32>, dim3((unsigned)((todo + CPB - 1) / CPB), (unsigned)B), dim3(256),
                           0, stream, K, L, cend, nc, first, Kbar);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_chunk_limits(int B, int64_t L, int64_t q_len, int64_t g, const int32_t *cend, int64_t nc,
                               int32_t *glim, hipStream_t stream)
{
    const int64_t n = (int64_t)B * ((q_len + g - 1) / g);
    hipLaunchKernelGGL(chunk_limits_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, B, L, q_len, g,
                       cend, nc, glim);
    return hipGetLastError();
}

hipError_t launch_chunk_expand(const ChunkExpandParams &prm, int64_t groups, hipStream_t stream)
{
    hipLaunchKernelGGL(chunk_expand_kernel, dim3((unsigned)groups), dim3(kExpandThreads), 0, stream, prm);
    return hipGetLastError();
}

hipError_t launch_chunk_adaptive(int D, int B, const ChunkAdaptParams &prm, hipStream_t stream)
{
    const int64_t units = prm.npair + (prm.nfull % 2);
    if (units > 0) {
        if (D == 128)
            hipLaunchKernelGGL(chunk_disp_kernel<128>, dim3((unsigned)units, (unsigned)B), dim3(128), 0, stream, prm);
        else if (D == 32)
            hipLaunchKernelGGL(chunk_disp_kernel<32>, dim3((unsigned)units, (unsigned)B), dim3(32), 0, stream, prm);
        else
            return hipErrorInvalidValue;
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    hipLaunchKernelGGL(chunk_greedy_kernel, dim3((unsigned)B), dim3(kAdaptThreads), 0, stream, prm);
    return hipGetLastError();
}

}  // namespace dsaidx
