// reduce.hip - the second kernel of split-K decode: merges partials
// (m_k, l_k, o_k) into the output row
//     out = sum_k e^(m_k - M) o_k / sum_k e^(m_k - M) l_k,  M = max_k m_k.
// The pages do not describe partitioned decode; the merge is the running
// max / running sum update of the online softmax in the kernel sketch of
// "vLLM 推理引擎源码级拆解" §2.3, applied once per piece instead of once per
// token.
//
// Where the entries of a row live depends on the split:
//   fixed partitions  entry k of row (s, hq) is partition k, k < ceil(L/P);
//   balanced          the row's KV-head stream was cut over chunks c0..c1 of
//                     the guided schedule (kernels.hpp); entry e is slot 0 or
//                     1 of chunk c0 + e (see decode_balanced.hip), found from
//                     the tile prefix and the header the decode call wrote.
//
// Work layout.  A row is served by WPR wavefronts (WPR = 1 for short rows, 4
// when rows have many entries).  Lane (kg = lane / 16, c = lane % 16) of wave
// `sub` owns output columns [c*CW, c*CW + CW) and the entries e = j, j + 4*WPR,
// j + 8*WPR, ... with slot j = 4*sub + kg; each entry's CW columns are one
// contiguous load, and the loads of four entries are issued together, the
// first four before M is known.  M and the denominator are computed by every
// wave from the m and l values (tiny); the per-slot sums meet through lane
// shuffles and, for WPR = 4, through LDS.
#include "common.hpp"
#include "kernels.hpp"

namespace pkv {
namespace {

constexpr int kWaves = 4;
constexpr int kUnroll = 4;

// Merges n >= 2 entries into one output row.  idx(e) maps entry e to its
// index in the m/l arrays (o rows at idx * D).
template <class O, int D, int WPR, class Idx>
__device__ inline void merge_row(const ReduceParams& p, int n, Idx idx, size_t row,
                                 int wave, int sub) {
    constexpr int CW = D / 16;                 // columns per lane
    constexpr int SLOTS = 4 * WPR;             // entry slots per row
    typedef float colv __attribute__((ext_vector_type(CW)));
    __shared__ colv part_sum[WPR > 1 ? kWaves : 1][16];

    const int lane = threadIdx.x & 63;
    const int kg = lane >> 4;
    const int c = lane & 15;
    const int j = 4 * sub + kg;

    // Everything a short row needs is requested before anything waits: the
    // first 64 (m, l) pairs and the first round of this lane's partial
    // outputs (which do not depend on M).  Out-of-range slots read entry 0
    // and get weight 0.
    const size_t i0 = lane < n ? idx(lane) : 0;
    const float m0 = lane < n ? p.ws_m[i0] : -INFINITY;
    const float l0 = lane < n ? p.ws_l[i0] : 0.0f;
    colv o[kUnroll];
    float mo[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; u++) {
        const int e = j + u * SLOTS;
        const size_t ie = idx(e < n ? e : 0);
        o[u] = *(const colv*)(p.ws_o + ie * D + c * CW);
        mo[u] = p.ws_m[ie];
    }

    // M and the denominator over all entries (lanes stride by 64).
    float M = m0;
    for (int e = lane + 64; e < n; e += 64) M = fmaxf(M, p.ws_m[idx(e)]);
    M = group_max<64>(M);
    const float Ml = M * kLog2e;
    float den = lane < n ? exp2f(fmaf(m0, kLog2e, -Ml)) * l0 : 0.0f;
    for (int e = lane + 64; e < n; e += 64) {
        const size_t ie = idx(e);
        den += exp2f(fmaf(p.ws_m[ie], kLog2e, -Ml)) * p.ws_l[ie];
    }
    den = group_sum<64>(den);

    // Weighted sum of this lane's slot over its columns, kUnroll entries per
    // round.
    colv acc = colv{};
    for (int e0 = j; e0 < n; e0 += SLOTS * kUnroll) {
        if (e0 != j) {
#pragma unroll
            for (int u = 0; u < kUnroll; u++) {
                const int e = e0 + u * SLOTS;
                const size_t ie = idx(e < n ? e : 0);
                o[u] = *(const colv*)(p.ws_o + ie * D + c * CW);
                mo[u] = p.ws_m[ie];
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; u++) {
            const int e = e0 + u * SLOTS;
            const float w = e < n ? exp2f(fmaf(mo[u], kLog2e, -Ml)) : 0.0f;
#pragma unroll
            for (int q = 0; q < CW; q++) acc[q] = fmaf(w, o[u][q], acc[q]);
        }
    }
    // Combine the four slots of this wave (lanes c, c+16, c+32, c+48).
#pragma unroll
    for (int q = 0; q < CW; q++) acc[q] = strided_sum<16>(acc[q]);
    if constexpr (WPR > 1) {
        if (kg == 0) part_sum[wave][c] = acc;
        __syncthreads();
        if (wave != 0 || kg != 0) return;
#pragma unroll
        for (int w = 1; w < WPR; w++) {
            const colv x = part_sum[w][c];
#pragma unroll
            for (int q = 0; q < CW; q++) acc[q] += x[q];
        }
    } else {
        if (kg != 0) return;
    }
    const float inv = 1.0f / den;
    typedef typename O::T OT;
    typedef OT ovec __attribute__((ext_vector_type(CW)));
    ovec r;
#pragma unroll
    for (int q = 0; q < CW; q++) r[q] = O::narrow(acc[q] * inv);
    *(ovec*)((OT*)p.out + row * D + c * CW) = r;
}

// ---- fixed partitions -------------------------------------------------------

template <class O, int D, int WPR>
__global__ __launch_bounds__(64 * kWaves) void reduce_kernel(ReduceParams p) {
    constexpr int RPB = kWaves / WPR;          // rows per workgroup
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int sub = wave % WPR;
    const int row = blockIdx.x * RPB + wave / WPR;   // s * Hq + hq
    // With WPR > 1 a workgroup is one row, so these exits are workgroup-uniform.
    if (row >= p.S * p.Hq) return;
    const int s = row / p.Hq;
    int L = p.lens[s];
    L = L < p.len_cap ? L : p.len_cap;
    const int nparts = L > 0 ? (L + p.P - 1) / p.P : 0;
    if (nparts <= 1) return;
    const size_t base = (size_t)row * p.P_max;
    merge_row<O, D, WPR>(p, nparts, [&](int k) { return base + (size_t)k; }, (size_t)row, wave,
                         sub);
}

// ---- balanced split ---------------------------------------------------------

// MULTI: rows of a balanced multi-query call, numbered (sequence s, query
// token j < max_query_len of it, head) so that no search maps a row to its
// sequence; the output row is (query_start[s] + j, head).  A token's column
// in its stream is j * G + head % G, and a token placed before its sequence
// (its column saw nothing) gets a zero row.
template <class O, int D, int WPR, bool MULTI>
__global__ __launch_bounds__(64 * kWaves) void reduce_balanced_kernel(ReduceParams p) {
    constexpr int RPB = kWaves / WPR;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int sub = wave % WPR;
    const int row = blockIdx.x * RPB + wave / WPR;
    const int32_t* hdr = p.ws_hdr;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        // The decode kernel is done with the chunk counter: return it to 0,
        // below any call's base, so that the next call takes it over even
        // when it carries the same call number (a replayed graph freezes
        // the number in the kernel's arguments).
        *(unsigned long long*)(const_cast<int32_t*>(hdr) + kHdrCounter) = 0ull;
    }
    if (row >= p.S * p.Hq) return;
    const int nW = hdr[kHdrNW];
    const int Hkv = hdr[kHdrHkv];
    const int G = hdr[kHdrG];
    const int T = hdr[kHdrT];
    const int S = MULTI ? p.S_seq : p.S;
    // A workspace not written by a balanced call of this shape: write
    // nothing rather than follow its indices.
    if (hdr[kHdrMagic] != kBalancedMagic || nW < 1 || nW > kBalancedMaxWaves || G < 1 ||
        Hkv != p.Hkv || Hkv * G != p.Hq || T < 0 || p.ws_pre[S] != T)
        return;
    const Sched q = make_sched(T, nW);
    const int hq = row % p.Hq;
    const int h = hq / G;
    int s = row / p.Hq, col = hq % G, ncol = G;
    size_t orow = (size_t)row;                  // output row
    typedef typename O::T OT;
    auto zero_row = [&]() {
        if (sub == 0)
            for (int d = lane; d < D; d += 64) ((OT*)p.out)[orow * D + d] = O::narrow(0.0f);
    };
    if constexpr (MULTI) {
        const int maxq = p.S / S;               // p.S = num_seqs * max_query_len
        s = row / (maxq * p.Hq);
        const int j = (row / p.Hq) % maxq;
        const int QPG = 16 / G;
        const int q0 = p.q_start[s];
        const int n = min(p.q_start[s + 1] - q0, QPG);
        if (j >= n) return;                     // no such query token
        orow = (size_t)(q0 + j) * p.Hq + hq;
        col = j * G + hq % G;
        ncol = QPG * G;
        int L = p.lens[s];
        L = L < p.len_cap ? L : p.len_cap;
        if (L - n + j < 0) {                    // its column saw no token
            zero_row();
            return;
        }
    }
    const int p0 = p.ws_pre[s], p1 = p.ws_pre[s + 1];
    if (p0 < 0 || p1 < p0 || p1 > T || (p1 - p0) % Hkv != 0) return;
    const int nt = (p1 - p0) / Hkv;
    if (nt == 0) {                              // no tokens: a zero row
        zero_row();
        return;
    }
    const int g0 = p0 + h * nt;                 // first tile of stream (s, h)
    const int c0 = chunk_of(q, g0);
    const int c1 = chunk_of(q, g0 + nt - 1);
    if (c0 == c1) return;                       // one chunk held it: decode wrote the row
    const int slot0 = chunk_begin(q, c0) < g0 ? 1 : 0;
    merge_row<O, D, WPR>(
        p, c1 - c0 + 1,
        [&](int e) {
            const int slot = e == 0 ? slot0 : 0;
            return ((size_t)(c0 + e) * 2 + slot) * ncol + col;
        },
        orow, wave, sub);
}

template <class O, int D, bool BAL>
hipError_t launch_w(const ReduceParams& p, bool wide, hipStream_t st) {
    const long rows = (long)p.S * p.Hq;
    const dim3 block(64 * kWaves);
    if (wide) {
        const dim3 grid((unsigned)rows);
        if (BAL && p.q_start)
            return launch_kernel(reduce_balanced_kernel<O, D, 4, true>, grid, block, st, p);
        if (BAL) return launch_kernel(reduce_balanced_kernel<O, D, 4, false>, grid, block, st, p);
        return launch_kernel(reduce_kernel<O, D, 4>, grid, block, st, p);
    }
    const dim3 grid((unsigned)((rows + kWaves - 1) / kWaves));
    if (BAL && p.q_start)
        return launch_kernel(reduce_balanced_kernel<O, D, 1, true>, grid, block, st, p);
    if (BAL) return launch_kernel(reduce_balanced_kernel<O, D, 1, false>, grid, block, st, p);
    return launch_kernel(reduce_kernel<O, D, 1>, grid, block, st, p);
}

template <class O, bool BAL>
hipError_t launch_d(const ReduceParams& p, bool wide, hipStream_t st) {
    if (p.D == 64) return launch_w<O, 64, BAL>(p, wide, st);
    if (p.D == 128) return launch_w<O, 128, BAL>(p, wide, st);
    return hipErrorInvalidValue;
}

template <bool BAL>
hipError_t launch_o(int out_dt, const ReduceParams& p, bool wide, hipStream_t st) {
    switch (out_dt) {
    case kF32: return launch_d<F32, BAL>(p, wide, st);
    case kF16: return launch_d<F16, BAL>(p, wide, st);
    case kBF16: return launch_d<BF16, BAL>(p, wide, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_reduce(int out_dt, const ReduceParams& p, hipStream_t st) {
    return launch_o<false>(out_dt, p, p.P_max > 32, st);
}

hipError_t launch_reduce_balanced(int out_dt, const ReduceParams& p, hipStream_t st) {
    // Few rows (long contexts, each row split over many waves): four waves
    // per row.
    return launch_o<true>(out_dt, p, (long)p.S * p.Hq <= 2048, st);
}

}  // namespace pkv
