// device.h - gfx950 building blocks shared by the indexer kernels: MFMA
// operand types, order-preserving score keys, wave-level ballots/prefix counts
// and the exact three-level radix cut used by every top-k / top-c.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsaidx {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// Word 3 of a raw buffer resource on this GPU family (no format conversion,
// plain byte addressing with a stride of 0).
constexpr int kBufferRsrcWord3 = 0x00020000;

// Register/LDS geometry of one query row (H heads of D dims) on the
// v_mfma_f32_32x32x16_bf16 tile: heads are MFMA rows, keys MFMA columns.
template <int H, int D>
struct Shape {
    static constexpr int MB = (H + 31) / 32;  // 32-head blocks (MFMA M)
    static constexpr int KS = D / 16;         // 16-deep MFMA K-steps
    static constexpr int ROWB = 2 * D;        // bytes of one bf16 key row
    static constexpr int ROWS = ROWB + 16;    // padded LDS row stride (bank spread)
    static constexpr int CHUNKS = ROWB / 16;  // 16-byte chunks per key row
};

// ---------------------------------------------------------------- score keys
// A selection ranks keys by (score descending, index ascending). A score is
// turned into an unsigned "key" that orders like the float (every finite
// value, -0 folded into +0 before the conversion); equal keys are broken by
// index, which the kernels get for free because they visit keys in
// ascending index order.
__device__ __forceinline__ uint32_t score_key(float f)
{
    uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_score(uint32_t k)
{
    uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
    return __uint_as_float(u);
}

// Level-1 bins are the top 11 bits of the key (sign, exponent, two mantissa
// bits); level 2 the next 11 bits, level 3 the last 10.
constexpr int kBins1 = 2048;
constexpr int kBins2 = 2048;
constexpr int kBins3 = 1024;

__device__ __forceinline__ uint32_t bin1(uint32_t key) { return key >> 21; }

// Smallest score of level-1 bin b (bins below 4 hold -inf and NaN patterns).
__device__ __forceinline__ float bin1_floor(int b)
{
    return b < 4 ? -__builtin_inff() : key_score((uint32_t)b << 21);
}

// max(0, x) as one v_max_i32 on the bit pattern: a finite float with the sign
// bit set is a negative int and becomes +0; any other float keeps its bits.
// (An fmaxf would first canonicalise x for IEEE NaN semantics: two VALU ops.)
__device__ __forceinline__ float relu(float x)
{
    return __int_as_float(max(__float_as_int(x), 0));
}

// ---------------------------------------------------------------- wave tools
__device__ __forceinline__ int lane_id() { return __lane_id(); }

// number of set bits of m below the calling lane
__device__ __forceinline__ int prefix_count(uint64_t m)
{
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Sum of the two half-waves: lane l and lane l^32 both get v[l%32] + v[l%32+32]
// (added in that order in every lane, so both halves hold the same bits).
__device__ __forceinline__ float half_wave_sum(float v)
{
    // With both operands equal, the swap returns (v[l%32], v[l%32+32]) in
    // every lane l.
    auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// Two such sums at once: lane l < 32 gets a[l] + a[l+32], lane l >= 32 gets
// b[l-32] + b[l] (the lower half's value first in both, as above). The swap
// exchanges the upper half of its first operand with the lower half of its
// second, leaving (a[l], b[l-32]) and (a[l+32], b[l]) per lane.
__device__ __forceinline__ float half_wave_sum2(float a, float b)
{
    auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// Issue priority of the calling wave, 0 (lowest) to 3, from a value the
// compiler knows once loops are unrolled (s_setprio takes an immediate).
__device__ __forceinline__ void wave_priority(int p)
{
    if (p >= 3)
        __builtin_amdgcn_s_setprio(3);
    else if (p == 2)
        __builtin_amdgcn_s_setprio(2);
    else if (p == 1)
        __builtin_amdgcn_s_setprio(1);
    else
        __builtin_amdgcn_s_setprio(0);
}

// v moved across the lanes of each 16-lane row by a DPP control (gfx9
// encoding); lanes whose source lies outside the row get `old`.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t old, uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, 0xF, 0xF, false);
}

// Wave-wide reduction by a commutative, associative op; every lane gets the
// result. Butterflies inside each quad and each row are DPP operands of the
// op itself; the rows, then the halves, are combined by lane swaps. No LDS
// round trip. Every lane of the wave must be active.
template <typename Op>
__device__ __forceinline__ uint32_t wave_reduce(uint32_t v, Op op)
{
    v = op(v, dpp_u32<0xB1>(v, v));   // quad_perm [1,0,3,2]
    v = op(v, dpp_u32<0x4E>(v, v));   // quad_perm [2,3,0,1]
    v = op(v, dpp_u32<0x141>(v, v));  // row_half_mirror: the other quad of 8
    v = op(v, dpp_u32<0x140>(v, v));  // row_mirror: the other 8 of 16
    const auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    v = op(p[0], p[1]);               // rows 0+1, rows 2+3
    const auto q = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return op(q[0], q[1]);            // both halves
}

// Wave-wide sum of an int (all lanes get it).
__device__ __forceinline__ int wave_sum(int v)
{
    return (int)wave_reduce((uint32_t)v, [](uint32_t a, uint32_t b) { return a + b; });
}

__device__ __forceinline__ uint32_t wave_min(uint32_t v)
{
    return wave_reduce(v, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
}

__device__ __forceinline__ uint32_t wave_max(uint32_t v)
{
    return wave_reduce(v, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
}

// ---------------------------------------------------------------- radix cut
// A cut describes the selected set of a scored list: an entry is in when its
// key is above kgt, or equal to keq and among the first req such entries in
// index order.
struct Cut {
    int64_t kgt;
    uint32_t keq;
    int req;
};

// Inclusive suffix sum over the lanes of a wave: lane l gets sum_{l' >= l} v.
// Within each row of 16 lanes a shift-and-add ladder (DPP row shifts, zero
// past the row's end); then each row adds the totals of the rows above it,
// read from their first lanes. Every lane of the wave must be active.
__device__ __forceinline__ int wave_suffix_sum(int v)
{
    const int l = lane_id();
    v += (int)dpp_u32<0x101>(0u, (uint32_t)v);  // row_shl:1
    v += (int)dpp_u32<0x102>(0u, (uint32_t)v);  // row_shl:2
    v += (int)dpp_u32<0x104>(0u, (uint32_t)v);  // row_shl:4
    v += (int)dpp_u32<0x108>(0u, (uint32_t)v);  // row_shl:8
    const int t1 = __builtin_amdgcn_readlane(v, 16);
    const int t2 = __builtin_amdgcn_readlane(v, 32);
    const int t3 = __builtin_amdgcn_readlane(v, 48);
    return v + (l < 16 ? t1 : 0) + (l < 32 ? t2 : 0) + (l < 48 ? t3 : 0);
}

// Largest bin x with sum_{y >= x} h[y] >= target (the caller guarantees the
// total reaches target); above = sum_{y > x} h[y]. NB is a multiple of 64.
// One wave; h is an LDS histogram; the result is wave-uniform. Lane l first
// sums bins [l*P, (l+1)*P); the crossing lane's bins are then resolved 64 at
// a time, top down, with a wave suffix scan (no serial walk).
template <int NB>
__device__ __forceinline__ void find_bin(const uint32_t *h, int target, int &x, int &above)
{
    constexpr int P = NB / kWave;
    const int l = lane_id();
    int s = 0;
#pragma unroll
    for (int p = 0; p < P; ++p)
        s += (int)h[l * P + p];
    const int t = wave_suffix_sum(s);
    const uint64_t m = ballot(t >= target);
    const int lc = 63 - __builtin_clzll(m);  // highest lane whose suffix reaches target
    int run = __builtin_amdgcn_readlane(t, lc) - __builtin_amdgcn_readlane(s, lc);
    int bx = lc * P, ab = run;
    for (int top = P; top > 0; top -= kWave) {
        const int lo = top > kWave ? top - kWave : 0;  // bins [lo, top) of lane lc's range
        const int i = lo + l;
        const int v = (i < top) ? (int)h[lc * P + i] : 0;
        const int sv = wave_suffix_sum(v) + run;    // run + sum of bins [i, top)
        const uint64_t mm = ballot(i < top && sv >= target);
        if (mm) {
            const int li = 63 - __builtin_clzll(mm);
            bx = lc * P + lo + li;
            ab = __builtin_amdgcn_readlane(sv - v, li);
            break;
        }
        run = __builtin_amdgcn_readlane(sv, 0);  // all of [lo, top) added
    }
    x = uniform(bx);
    above = uniform(ab);
}

// Workgroup barrier for LDS traffic only: each wave waits for its own LDS
// operations, not for its global stores (a __syncthreads would also wait for
// those, microseconds after a burst of stores). The memory clobber keeps the
// compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_sync()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int NB>
__device__ __forceinline__ void clear_hist(uint32_t *h)
{
#pragma unroll
    for (int p = 0; p < NB / kWave; ++p)
        h[p * kWave + lane_id()] = 0u;
}

}  // namespace dsaidx
