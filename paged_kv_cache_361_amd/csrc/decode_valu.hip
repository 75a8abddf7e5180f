// decode_valu.hip - paged decode attention on the vector ALUs.
//
// The general kernel of the library: every supported (query, cache) type
// pair, head_dim 64/128, any block size, GQA groups up to 8.  It follows the
// single-query kernel of "vLLM 推理引擎源码级拆解" §2.3 (logical block =
// t / bs, offset = t % bs, physical block from the table, dot with the
// query, online softmax) with the work laid out for 64-lane wavefronts:
//
//  * One wavefront owns one unit = (sequence, KV head, partition) and all G
//    query heads that share the KV head, so each K/V row is read from HBM
//    once per group.  A workgroup is four independent wavefronts.
//  * A token row (D elements of one KV head) is spread over R lanes, each
//    holding a CH-element chunk loaded with one 16-byte (8-byte for fp8)
//    load, so 64/R tokens are fetched per load instruction and all bytes of a
//    row are contiguous across neighbouring lanes.
//  * Tiles of 16 tokens: scores by a per-lane partial dot product and a
//    reduction over the R lanes of a row; the running max is kept uniform
//    across the wavefront so the per-lane PV accumulators can simply be
//    summed at the end.
//  * Lanes past the end of the range re-read the last live token instead of
//    whatever the pool holds there, and their weight is forced to zero, so
//    poisoned slots and table padding are never touched.
#include "common.hpp"
#include "kernels.hpp"

namespace pkv {
namespace {

constexpr int kWaves = 4;

template <class Q, class C, int D, int GMAX>
__global__ __launch_bounds__(64 * kWaves) void decode_valu_kernel(DecodeParams p) {
    typedef typename C::T CT;
    typedef typename Q::T QT;
    constexpr int E = C::kBytes;
    constexpr int CH = (E == 4) ? 4 : 8;           // elements per lane per load
    constexpr int R = D / CH;                      // lanes per token row
    constexpr int TPL = 64 / R;                    // tokens per load
    constexpr int TILE = TPL >= 16 ? TPL : 16;
    constexpr int U = TILE / TPL;                  // loads per tile (K and V each)
    static_assert(D % CH == 0 && 64 % R == 0, "row must tile a wavefront");
    typedef CT cvec __attribute__((ext_vector_type(CH)));
    typedef QT qvec __attribute__((ext_vector_type(CH)));

    const int lane = threadIdx.x & 63;
    const int unit = blockIdx.x * kWaves + (threadIdx.x >> 6);
    const int h = unit % p.Hkv;
    const int rest = unit / p.Hkv;
    const int part = rest % p.P_max;
    const int s = rest / p.P_max;
    if (s >= p.S) return;

    const int G = p.G;
    int L = p.lens[s];
    L = L < p.len_cap ? L : p.len_cap;
    const int c = lane % R;
    const int r = lane / R;
    const size_t qrow0 = ((size_t)s * p.Hq + (size_t)h * G) * D;

    int t_begin = 0, t_end = L;
    bool final_out = true;
    if (p.P > 0) {
        const int nparts = L > 0 ? (L + p.P - 1) / p.P : 0;
        t_begin = part * p.P;
        t_end = min(L, t_begin + p.P);
        final_out = nparts <= 1;
    }
    if (L <= 0) {
        if (part == 0 && r == 0) {
            for (int g = 0; g < G; g++)
                for (int e = 0; e < CH; e++)
                    ((QT*)p.out)[qrow0 + (size_t)g * D + c * CH + e] = Q::narrow(0.0f);
        }
        return;
    }
    if (t_begin >= t_end) return;

    float qv[GMAX][CH];
#pragma unroll
    for (int g = 0; g < GMAX; g++) {
        if (g < G) {
            const qvec x = *(const qvec*)((const QT*)p.q + qrow0 + (size_t)g * D + c * CH);
#pragma unroll
            for (int e = 0; e < CH; e++) qv[g][e] = Q::widen(x[e]);
        } else {
#pragma unroll
            for (int e = 0; e < CH; e++) qv[g][e] = 0.0f;
        }
    }

    const size_t row_stride = (size_t)p.Hkv * D;   // elements between slots
    const CT* kbase = (const CT*)p.k + (size_t)h * D + c * CH;
    const CT* vbase = (const CT*)p.v + (size_t)h * D + c * CH;
    const int32_t* table = p.tables + (size_t)s * p.max_blocks;
    const uint32_t nb_last = (uint32_t)p.NB - 1u;

    float m[GMAX], lsum[GMAX], acc[GMAX][CH];
#pragma unroll
    for (int g = 0; g < GMAX; g++) {
        m[g] = -INFINITY;
        lsum[g] = 0.0f;
#pragma unroll
        for (int e = 0; e < CH; e++) acc[g][e] = 0.0f;
    }

    for (int t0 = t_begin; t0 < t_end; t0 += TILE) {
        cvec kr[U], vr[U];
        bool live[U];
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int t = t0 + u * TPL + r;
            live[u] = t < t_end;
            const int tl = live[u] ? t : t_end - 1;
            uint32_t phys = (uint32_t)table[tl / p.bs];
            phys = phys < nb_last ? phys : nb_last;
            const size_t off = ((size_t)phys * p.bs + (size_t)(tl % p.bs)) * row_stride;
            kr[u] = *(const cvec*)(kbase + off);
            vr[u] = *(const cvec*)(vbase + off);
        }
        float z[U][GMAX];
#pragma unroll
        for (int u = 0; u < U; u++) {
            float kf[CH];
#pragma unroll
            for (int e = 0; e < CH; e++) kf[e] = C::widen(kr[u][e]);
#pragma unroll
            for (int g = 0; g < GMAX; g++) {
                float d = 0.0f;
#pragma unroll
                for (int e = 0; e < CH; e++) d = fmaf(qv[g][e], kf[e], d);
                d = group_sum<R>(d) * p.scale_log2;
                z[u][g] = live[u] ? d : -INFINITY;
            }
        }
#pragma unroll
        for (int g = 0; g < GMAX; g++) {
            float mx = z[0][g];
#pragma unroll
            for (int u = 1; u < U; u++) mx = fmaxf(mx, z[u][g]);
            mx = strided_max<R>(mx);
            const float m_new = fmaxf(m[g], mx);
            if (m_new > m[g]) {                     // uniform across the wave
                const float alpha = exp2f(m[g] - m_new);
                lsum[g] *= alpha;
#pragma unroll
                for (int e = 0; e < CH; e++) acc[g][e] *= alpha;
                m[g] = m_new;
            }
        }
#pragma unroll
        for (int u = 0; u < U; u++) {
            float vf[CH];
#pragma unroll
            for (int e = 0; e < CH; e++) vf[e] = C::widen(vr[u][e]);
#pragma unroll
            for (int g = 0; g < GMAX; g++) {
                const float w = exp2f(z[u][g] - m[g]);   // 0 for dead lanes
                lsum[g] += w;
#pragma unroll
                for (int e = 0; e < CH; e++) acc[g][e] = fmaf(w, vf[e], acc[g][e]);
            }
        }
    }

    // Combine the row groups: every lane of a group holds the same weights,
    // so the per-group sums add up to the wavefront total.
#pragma unroll
    for (int g = 0; g < GMAX; g++) {
        lsum[g] = strided_sum<R>(lsum[g]);
#pragma unroll
        for (int e = 0; e < CH; e++) acc[g][e] = strided_sum<R>(acc[g][e]);
    }
    if (r != 0) return;
#pragma unroll
    for (int g = 0; g < GMAX; g++) {
        if (g >= G) break;
        if (final_out) {
            const float inv = p.v_scale / lsum[g];
            qvec o;
#pragma unroll
            for (int e = 0; e < CH; e++) o[e] = Q::narrow(acc[g][e] * inv);
            *(qvec*)((QT*)p.out + qrow0 + (size_t)g * D + c * CH) = o;
        } else {
            const size_t idx = ((size_t)s * p.Hq + (size_t)h * G + g) * p.P_max + part;
            if (c == 0) {
                p.ws_m[idx] = m[g] * kLn2;
                p.ws_l[idx] = lsum[g];
            }
            float* o = p.ws_o + idx * D + c * CH;
#pragma unroll
            for (int e = 0; e < CH; e++) o[e] = acc[g][e] * p.v_scale;
        }
    }
}

template <class Q, class C, int D, int GMAX>
hipError_t launch_one(const DecodeParams& p, hipStream_t st) {
    const long units = (long)p.S * p.P_max * p.Hkv;
    const dim3 grid((unsigned)((units + kWaves - 1) / kWaves)), block(64 * kWaves);
    return launch_kernel(decode_valu_kernel<Q, C, D, GMAX>, grid, block, st, p);
}

template <class Q, class C, int D>
hipError_t launch_g(const DecodeParams& p, hipStream_t st) {
    if (p.G <= 1) return launch_one<Q, C, D, 1>(p, st);
    if (p.G <= 2) return launch_one<Q, C, D, 2>(p, st);
    if (p.G <= 4) return launch_one<Q, C, D, 4>(p, st);
    if (p.G <= 8) return launch_one<Q, C, D, 8>(p, st);
    return hipErrorInvalidValue;
}

template <class Q, class C>
hipError_t launch_d(const DecodeParams& p, hipStream_t st) {
    if (p.D == 64) return launch_g<Q, C, 64>(p, st);
    if (p.D == 128) return launch_g<Q, C, 128>(p, st);
    return hipErrorInvalidValue;
}

}  // namespace

bool decode_valu_supported(int qdt, int cdt, int D, int G) {
    const bool types = (qdt == cdt && qdt != kFP8) ||
                       (cdt == kFP8 && (qdt == kF16 || qdt == kBF16));
    return types && (D == 64 || D == 128) && G >= 1 && G <= 8;
}

hipError_t launch_decode_valu(int qdt, int cdt, const DecodeParams& p, hipStream_t st) {
    if (!decode_valu_supported(qdt, cdt, p.D, p.G)) return hipErrorInvalidValue;
    if (cdt == kFP8) {
        if (qdt == kF16) return launch_d<F16, FP8>(p, st);
        return launch_d<BF16, FP8>(p, st);
    }
    switch (qdt) {
    case kF32: return launch_d<F32, F32>(p, st);
    case kF16: return launch_d<F16, F16>(p, st);
    case kBF16: return launch_d<BF16, BF16>(p, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace pkv
