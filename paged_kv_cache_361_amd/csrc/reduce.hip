// reduce.hip - the second kernel of split-K decode: merges per-partition
// partials (m_k, l_k, o_k) into the output row
//     out = sum_k e^(m_k - M) o_k / sum_k e^(m_k - M) l_k,  M = max_k m_k.
// The pages do not describe partitioned decode; the merge is the running
// max / running sum update of the online softmax in the kernel sketch of
// "vLLM 推理引擎源码级拆解" §2.3, applied once per partition instead of once
// per token.
//
// One wavefront per (sequence, query head): the maximum over partitions is a
// lane-parallel max; then, k ascending, every lane forms the (uniform) weight
// e^(m_k - M) and accumulates its D/64 output columns and the denominator.
#include "common.hpp"
#include "kernels.hpp"

namespace pkv {
namespace {

constexpr int kWaves = 4;

template <class O, int D>
__global__ __launch_bounds__(64 * kWaves) void reduce_kernel(ReduceParams p) {
    constexpr int PER = D / 64;
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * kWaves + (threadIdx.x >> 6);   // s * Hq + hq
    if (row >= p.S * p.Hq) return;
    const int s = row / p.Hq;
    int L = p.lens[s];
    L = L < p.len_cap ? L : p.len_cap;
    const int nparts = L > 0 ? (L + p.P - 1) / p.P : 0;
    if (nparts <= 1) return;

    const size_t base = (size_t)row * p.P_max;
    float M = -INFINITY;
    for (int k = lane; k < nparts; k += 64) M = fmaxf(M, p.ws_m[base + k]);
    M = group_max<64>(M);
    float acc[PER];
#pragma unroll
    for (int j = 0; j < PER; j++) acc[j] = 0.0f;
    float den = 0.0f;
    const float* o = p.ws_o + base * D + lane * PER;
    for (int k = 0; k < nparts; k++) {
        const float wk = exp2f((p.ws_m[base + k] - M) * kLog2e);
        den = fmaf(wk, p.ws_l[base + k], den);
#pragma unroll
        for (int j = 0; j < PER; j++) acc[j] = fmaf(wk, o[(size_t)k * D + j], acc[j]);
    }
    const float inv = 1.0f / den;
    typename O::T* out = (typename O::T*)p.out + (size_t)row * D + lane * PER;
#pragma unroll
    for (int j = 0; j < PER; j++) out[j] = O::narrow(acc[j] * inv);
}

template <class O>
hipError_t launch_d(const ReduceParams& p, hipStream_t st) {
    const dim3 grid((unsigned)((p.S * (long)p.Hq + kWaves - 1) / kWaves)), block(64 * kWaves);
    if (p.D == 64) return launch_kernel(reduce_kernel<O, 64>, grid, block, st, p);
    if (p.D == 128) return launch_kernel(reduce_kernel<O, 128>, grid, block, st, p);
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
