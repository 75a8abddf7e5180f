// reduce.hip - the second kernel of split-K decode: merges per-partition
// partials (m_k, l_k, o_k) into the output row
//     out = sum_k e^(m_k - M) o_k / sum_k e^(m_k - M) l_k,  M = max_k m_k.
// The pages do not describe partitioned decode; the merge is the running
// max / running sum update of the online softmax in the kernel sketch of
// "vLLM 推理引擎源码级拆解" §2.3, applied once per partition instead of once
// per token.
//
// Work layout.  A row (sequence, query head) is served by WPR wavefronts
// (WPR = 1 for short rows, 4 when rows have many partitions).  Lane
// (kg = lane / 16, c = lane % 16) of wave `sub` owns output columns
// [c*CW, c*CW + CW) and the partitions k = j, j + 4*WPR, j + 8*WPR, ... with
// slot j = 4*sub + kg; each partition's CW columns are one contiguous load,
// and the loads of four partitions are issued together.  M and the
// denominator are computed by every wave from the m_k and l_k arrays (tiny);
// the per-slot sums meet through lane shuffles and, for WPR = 4, through LDS.
#include "common.hpp"
#include "kernels.hpp"

namespace pkv {
namespace {

constexpr int kWaves = 4;
constexpr int kUnroll = 4;

template <class O, int D, int WPR>
__global__ __launch_bounds__(64 * kWaves) void reduce_kernel(ReduceParams p) {
    constexpr int CW = D / 16;                 // columns per lane
    constexpr int SLOTS = 4 * WPR;             // partition slots per row
    constexpr int RPB = kWaves / WPR;          // rows per workgroup
    typedef float colv __attribute__((ext_vector_type(CW)));
    __shared__ colv part_sum[WPR > 1 ? kWaves : 1][16];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int sub = wave % WPR;
    const int row = blockIdx.x * RPB + wave / WPR;   // s * Hq + hq
    const int rows = p.S * p.Hq;
    // With WPR > 1 a workgroup is one row, so these exits are workgroup-uniform.
    if (row >= rows) return;
    const int s = row / p.Hq;
    int L = p.lens[s];
    L = L < p.len_cap ? L : p.len_cap;
    const int nparts = L > 0 ? (L + p.P - 1) / p.P : 0;
    if (nparts <= 1) return;

    const size_t base = (size_t)row * p.P_max;
    const float* ms = p.ws_m + base;
    const float* ls = p.ws_l + base;

    // M and the denominator, over all partitions (lanes stride by 64).
    float M = -INFINITY;
    for (int k = lane; k < nparts; k += 64) M = fmaxf(M, ms[k]);
    M = group_max<64>(M);
    const float Ml = M * kLog2e;
    float den = 0.0f;
    for (int k = lane; k < nparts; k += 64) den += exp2f(fmaf(ms[k], kLog2e, -Ml)) * ls[k];
    den = group_sum<64>(den);

    // Weighted sum of this lane's slot over its columns.
    const int kg = lane >> 4;
    const int c = lane & 15;
    const int j = 4 * sub + kg;
    const float* ob = p.ws_o + base * D + c * CW;
    colv acc = colv{};
    for (int k0 = j; k0 < nparts; k0 += SLOTS * kUnroll) {
        colv o[kUnroll];
        float m[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; u++) {
            const int k = k0 + u * SLOTS;
            const int kk = k < nparts ? k : j;             // in range; weight zeroed below
            o[u] = *(const colv*)(ob + (size_t)kk * D);
            m[u] = ms[kk];
        }
#pragma unroll
        for (int u = 0; u < kUnroll; u++) {
            const int k = k0 + u * SLOTS;
            const float w = k < nparts ? exp2f(fmaf(m[u], kLog2e, -Ml)) : 0.0f;
#pragma unroll
            for (int e = 0; e < CW; e++) acc[e] = fmaf(w, o[u][e], acc[e]);
        }
    }
    // Combine the four slots of this wave (lanes c, c+16, c+32, c+48).
#pragma unroll
    for (int e = 0; e < CW; e++) acc[e] = strided_sum<16>(acc[e]);
    if constexpr (WPR > 1) {
        if (kg == 0) part_sum[wave][c] = acc;
        __syncthreads();
        if (wave != 0 || kg != 0) return;
#pragma unroll
        for (int w = 1; w < WPR; w++) {
            const colv x = part_sum[w][c];
#pragma unroll
            for (int e = 0; e < CW; e++) acc[e] += x[e];
        }
    } else {
        if (kg != 0) return;
    }
    const float inv = 1.0f / den;
    typedef typename O::T OT;
    typedef OT ovec __attribute__((ext_vector_type(CW)));
    ovec r;
#pragma unroll
    for (int e = 0; e < CW; e++) r[e] = O::narrow(acc[e] * inv);
    *(ovec*)((OT*)p.out + (size_t)row * D + c * CW) = r;
}

template <class O, int D>
hipError_t launch_w(const ReduceParams& p, hipStream_t st) {
    const long rows = (long)p.S * p.Hq;
    const dim3 block(64 * kWaves);
    if (p.P_max > 32) {
        const dim3 grid((unsigned)rows);
        return launch_kernel(reduce_kernel<O, D, 4>, grid, block, st, p);
    }
    const dim3 grid((unsigned)((rows + kWaves - 1) / kWaves));
    return launch_kernel(reduce_kernel<O, D, 1>, grid, block, st, p);
}

template <class O>
hipError_t launch_d(const ReduceParams& p, hipStream_t st) {
    if (p.D == 64) return launch_w<O, 64>(p, st);
    if (p.D == 128) return launch_w<O, 128>(p, st);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_reduce(int out_dt, const ReduceParams& p, hipStream_t st) {
    switch (out_dt) {
    case kF32: return launch_d<F32>(p, st);
    case kF16: return launch_d<F16>(p, st);
    case kBF16: return launch_d<BF16>(p, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace pkv
