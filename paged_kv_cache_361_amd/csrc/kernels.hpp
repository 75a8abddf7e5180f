// kernels.hpp - internal launch interface between the C ABI (api.hip) and the
// kernel translation units.  Not installed; the public contract is
// include/pagedkv.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

enum DType : int { kF32 = 0, kF16 = 1, kBF16 = 2, kFP8 = 3 };

struct WriteParams {
    const void* key;
    const void* value;
    void* k_cache;
    void* v_cache;
    const int64_t* slot_mapping;
    int64_t num_slots;     // num_blocks * block_size
    int T, Hkv, D;
    int src_bytes;         // bytes per source element
    float k_scale, v_scale;
};

struct DecodeParams {
    void* out;
    const void* q;
    const void* k;
    const void* v;
    const int32_t* tables;
    const int32_t* lens;
    float* ws_m;           // split-K partials (nullptr in one-pass mode)
    float* ws_l;
    float* ws_o;
    int S, Hq, Hkv, D, G, bs, NB, max_blocks;
    int len_cap;           // min(max_seq_len, max_blocks * bs)
    int P;                 // partition size, 0 = one pass
    int P_max;             // partitions per sequence covered by the grid
    float scale_log2;      // scale * k_scale * log2(e): scores in base-2 units
    float v_scale;
};

struct ReduceParams {
    void* out;
    const float* ws_m;
    const float* ws_l;
    const float* ws_o;
    const int32_t* lens;
    int S, Hq, D, P, P_max, len_cap;
};

// Launches a kernel whose only parameter is a parameter struct and returns
// that launch's own status.
template <typename Kernel, typename Params>
inline hipError_t launch_kernel(Kernel kernel, dim3 grid, dim3 block, hipStream_t st,
                                const Params& p) {
    void* args[] = {const_cast<Params*>(&p)};
    return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, args, 0, st);
}

// Launchers; the caller has checked the matching *_supported() first.  They
// return hipErrorInvalidValue for a combination without a kernel.
hipError_t launch_reshape_and_cache(int src, int cache, const WriteParams& p, hipStream_t st);
bool decode_valu_supported(int qdt, int cdt, int D, int G);
hipError_t launch_decode_valu(int qdt, int cdt, const DecodeParams& p, hipStream_t st);
bool decode_mfma_supported(int qdt, int cdt, int D, int G);
hipError_t launch_decode_mfma(int qdt, int cdt, const DecodeParams& p, hipStream_t st);
hipError_t launch_reduce(int out_dt, const ReduceParams& p, hipStream_t st);

}  // namespace pkv
