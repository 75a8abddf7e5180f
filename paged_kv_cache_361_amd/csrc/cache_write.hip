// cache_write.hip - reshape_and_cache: store new tokens' K/V rows in their
// pool slots ("vLLM 推理引擎源码级拆解" §2.2: a new token fills the next slot of
// its sequence's last block; the slot number comes from the caller).
//
// One workgroup per token.  In the pool, all KV heads of one slot are
// contiguous ([block][offset][head][dim]), so each token is one contiguous
// Hkv*D-element row on both sides: the copy is 16-byte vector loads and
// stores, and the fp8 variant converts 8 elements per lane.
#include "common.hpp"
#include "kernels.hpp"

namespace pkv {
namespace {

constexpr int kThreads = 128;

// Same storage type: a bit copy, 16 bytes per lane per step.
__global__ __launch_bounds__(kThreads) void copy_rows_kernel(WriteParams p) {
    const int row_bytes = p.Hkv * p.D * p.src_bytes;
    const int64_t slot = p.slot_mapping[blockIdx.x];
    if (slot < 0 || slot >= p.num_slots) return;
    const size_t src0 = (size_t)blockIdx.x * row_bytes;
    const size_t dst0 = (size_t)slot * row_bytes;
    const char* ks = (const char*)p.key + src0;
    const char* vs = (const char*)p.value + src0;
    char* kd = (char*)p.k_cache + dst0;
    char* vd = (char*)p.v_cache + dst0;
    for (int b = threadIdx.x * 16; b < row_bytes; b += kThreads * 16) {
        u32x4 k = *(const u32x4*)(ks + b);
        u32x4 v = *(const u32x4*)(vs + b);
        *(u32x4*)(kd + b) = k;
        *(u32x4*)(vd + b) = v;
    }
}

// Source format -> E4M3: y = x / scale in IEEE fp32 (correctly rounded
// divide), then round-to-nearest-even with saturation.
template <class Src>
__global__ __launch_bounds__(kThreads) void quantize_rows_kernel(WriteParams p) {
    typedef typename Src::T T;
    typedef T vec8 __attribute__((ext_vector_type(8)));
    const int64_t slot = p.slot_mapping[blockIdx.x];
    if (slot < 0 || slot >= p.num_slots) return;
    const int row = p.Hkv * p.D;
    const T* ks = (const T*)p.key + (size_t)blockIdx.x * row;
    const T* vs = (const T*)p.value + (size_t)blockIdx.x * row;
    uint8_t* kd = (uint8_t*)p.k_cache + (size_t)slot * row;
    uint8_t* vd = (uint8_t*)p.v_cache + (size_t)slot * row;
    for (int e = threadIdx.x * 8; e < row; e += kThreads * 8) {
        vec8 k = *(const vec8*)(ks + e);
        vec8 v = *(const vec8*)(vs + e);
        u32x2 ko = {0u, 0u}, vo = {0u, 0u};
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const float qk = Src::widen(k[j]) / p.k_scale;
            const float qv = Src::widen(v[j]) / p.v_scale;
            ko[j / 4] |= e4m3_encode(qk) << (8 * (j % 4));
            vo[j / 4] |= e4m3_encode(qv) << (8 * (j % 4));
        }
        *(u32x2*)(kd + e) = ko;
        *(u32x2*)(vd + e) = vo;
    }
}

// Whole-block copies.  Inside one pool this is copy on write of a shared
// block ("vLLM 推理引擎源码级拆解" §2.1: before a sequence writes into a block
// other tables still point at, the block is copied and the writer's table
// takes the copy); between the device pool and a pool in pinned host memory
// it is swapping (§3.2: a preempted sequence's blocks move to host memory and
// back).  One workgroup per pair, both pools, 16-byte vector loads and
// stores; a pair with a block id outside its pool, or a copy of a block onto
// itself, is skipped.
constexpr int kCopyThreads = 256;

__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(CopyParams p) {
    const int i = blockIdx.x;
    const int32_t src = p.pairs[2 * i], dst = p.pairs[2 * i + 1];
    if (src < 0 || src >= p.src_blocks || dst < 0 || dst >= p.dst_blocks) return;
    if (p.sk == p.dk && src == dst) return;
    const size_t so = (size_t)src * p.block_bytes, d_o = (size_t)dst * p.block_bytes;
    const char* ks = (const char*)p.sk + so;
    const char* vs = (const char*)p.sv + so;
    char* kd = (char*)p.dk + d_o;
    char* vd = (char*)p.dv + d_o;
    for (uint32_t b = threadIdx.x * 16u; b < p.block_bytes; b += kCopyThreads * 16u) {
        const u32x4 k = *(const u32x4*)(ks + b);
        const u32x4 v = *(const u32x4*)(vs + b);
        *(u32x4*)(kd + b) = k;
        *(u32x4*)(vd + b) = v;
    }
}

}  // namespace

hipError_t launch_copy_blocks(const CopyParams& p, hipStream_t st) {
    if (p.n == 0) return hipSuccess;
    return launch_kernel(copy_blocks_kernel, dim3(p.n), dim3(kCopyThreads), st, p);
}

hipError_t launch_reshape_and_cache(int src, int cache, const WriteParams& p, hipStream_t st) {
    if (p.T == 0) return hipSuccess;
    const dim3 grid(p.T), block(kThreads);
    if (src == cache) return launch_kernel(copy_rows_kernel, grid, block, st, p);
    if (cache != kFP8) return hipErrorInvalidValue;
    switch (src) {
    case kF32: return launch_kernel(quantize_rows_kernel<F32>, grid, block, st, p);
    case kF16: return launch_kernel(quantize_rows_kernel<F16>, grid, block, st, p);
    case kBF16: return launch_kernel(quantize_rows_kernel<BF16>, grid, block, st, p);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace pkv
