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
// Work layout.  A row is served by WPR wavefronts (WPR = 1 for short rows,
// 4 or 8 when rows have many entries; with WPR > 1 a workgroup is one row).
// Lane (kg = lane / 16, c = lane % 16) of wave `sub` owns output columns
// [c*CW, c*CW + CW) of the entries e = j, j + 4*WPR, j + 8*WPR, ... with
// slot j = 4*sub + kg.
//   One wave (merge_short): the row max and the denominator come from one
//   (m, l) pair per lane by wave-wide reductions, and the slots' first four
//   entries are loaded at the same time; short rows need no more.
//   Several waves (merge_row): a slot keeps a running reference max, sum and
//   output over its entries (the online-softmax update of the decode, once
//   per entry), loading kBatch entries per round with all their loads issued
//   together, so a row of n entries takes ceil(n / (4 * WPR * kBatch))
//   rounds of memory latency; the slots then meet at the row's max through
//   lane shuffles and LDS.
#include "common.hpp"
#include "kernels.hpp"

namespace pkv {
namespace {

constexpr int kWaves = 4;      // waves per workgroup of one-wave rows

// Entries per slot that merge_row loads per round.
constexpr int kBatch = 8;

// Waves per SIMD each kernel is compiled to fit (a register budget): eight
// for one-wave rows, so that a batch of 8192 rows (2048 workgroups of four
// waves) is resident at once on 256 CUs; four for the wide rows (two
// workgroups of eight waves per CU: 512 long rows at once).
constexpr int waves_per_simd(int WPR) { return WPR > 1 ? 4 : 8; }

// Waves per workgroup of a kernel serving rows with WPR waves each.
constexpr int wg_waves(int WPR) { return WPR > 1 ? WPR : kWaves; }

// An entry's CW values of one lane, from its compact form (f16 means x and
// the stored l; see compact_exponent) back to the sums o = x 2^(e - 15) l.
template <int CW>
__device__ inline auto widen_entry(_Float16 __attribute__((ext_vector_type(CW))) h, float l) {
    typedef float colv __attribute__((ext_vector_type(CW)));
    const float f = compact_scale(l);
    colv o;
#pragma unroll
    for (int q = 0; q < CW; q++) o[q] = (float)h[q] * f;
    return o;
}

// Merges n >= 1 entries into one output row served by WPR > 1 waves (one
// workgroup).  idx(e) maps entry e to its index in the m/l arrays (o rows at
// idx * D; COMPACT: compact rows of D f16 values).  A row whose entries hold
// no weight (every m = -inf) is written as zeros.
template <class O, int D, int WPR, bool COMPACT, class Idx>
__device__ inline void merge_row(const ReduceParams& p, int n, Idx idx, size_t row, int sub) {
    static_assert(WPR > 1, "one-wave rows take merge_short");
    constexpr int CW = D / 16;                 // columns per lane
    constexpr int SLOTS = 4 * WPR;             // entry slots per row
    constexpr int NP = WPR;
    typedef float colv __attribute__((ext_vector_type(CW)));
    typedef _Float16 hcol __attribute__((ext_vector_type(CW)));
    __shared__ colv part_sum[NP][16];
    __shared__ float part_m[NP], part_l[NP];

    const int lane = threadIdx.x & 63;
    const int kg = lane >> 4;
    const int c = lane & 15;
    const int j = 4 * sub + kg;

    // Running state of this lane's slot: reference max (log2 units), the sum
    // of the entries' l and the output columns, both scaled to it.
    float m_run = -INFINITY, l_run = 0.0f;
    colv acc = colv{};
    for (int e0 = j; e0 < n; e0 += SLOTS * kBatch) {
        colv o[kBatch];
        hcol h[kBatch];
        float m[kBatch], l[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; u++) {     // the round's loads, all at once
            const int e = e0 + u * SLOTS;
            o[u] = colv{};                     // entries past n: no weight, no loads
            h[u] = hcol{};
            m[u] = -INFINITY;
            l[u] = 0.0f;
            if (e < n) {
                const size_t ie = idx(e);
                if constexpr (COMPACT) h[u] = *(const hcol*)((const _Float16*)p.ws_o + ie * D + c * CW);
                else o[u] = *(const colv*)(p.ws_o + ie * D + c * CW);
                m[u] = p.ws_m[ie];
                l[u] = p.ws_l[ie];
            }
        }
        // Keep every load of the round ahead of the arithmetic: otherwise the
        // scheduler issues the o loads only once the m values are back, which
        // costs a second memory round trip per round.
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (COMPACT) {
#pragma unroll
            for (int u = 0; u < kBatch; u++) o[u] = widen_entry<CW>(h[u], l[u]);
        }
        float bm = m_run;
#pragma unroll
        for (int u = 0; u < kBatch; u++) {
            m[u] *= kLog2e;
            bm = fmaxf(bm, m[u]);
        }
        const float ref = bm == -INFINITY ? 0.0f : bm;
        const float f = exp2f(m_run - ref);
        l_run *= f;
#pragma unroll
        for (int q = 0; q < CW; q++) acc[q] *= f;
#pragma unroll
        for (int u = 0; u < kBatch; u++) {
            const float w = exp2f(m[u] - ref);
            l_run = fmaf(w, l[u], l_run);
#pragma unroll
            for (int q = 0; q < CW; q++) acc[q] = fmaf(w, o[u][q], acc[q]);
        }
        m_run = bm;
    }

    // The row's max over all slots, then every slot rescaled to it and summed:
    // the four slots of a wave (lanes c, c+16, c+32, c+48) by lane shuffles,
    // the waves of a row through LDS.
    float M = group_max<64>(m_run);
    if (lane == 0) part_m[sub] = M;
    __syncthreads();
    M = part_m[0];
#pragma unroll
    for (int w = 1; w < WPR; w++) M = fmaxf(M, part_m[w]);
    const float f = exp2f(m_run - (M == -INFINITY ? 0.0f : M));
    float den = strided_sum<16>(l_run * f);
#pragma unroll
    for (int q = 0; q < CW; q++) acc[q] = strided_sum<16>(acc[q] * f);
    if (kg == 0) part_sum[sub][c] = acc;
    if (lane == 0) part_l[sub] = den;
    __syncthreads();
    if (sub != 0 || kg != 0) return;
#pragma unroll
    for (int w = 1; w < WPR; w++) {
        const colv x = part_sum[w][c];
#pragma unroll
        for (int q = 0; q < CW; q++) acc[q] += x[q];
        den += part_l[w];
    }
    const float inv = den > 0.0f ? 1.0f / den : 0.0f;
    typedef typename O::T OT;
    typedef OT ovec __attribute__((ext_vector_type(CW)));
    ovec r;
#pragma unroll
    for (int q = 0; q < CW; q++) r[q] = O::narrow(acc[q] * inv);
    *(ovec*)((OT*)p.out + row * D + c * CW) = r;
}

// merge_row for rows served by one wave (WPR = 1), with n up to a few dozen
// entries.  Everything such a row needs is requested before anything waits:
// the first 64 (m, l) pairs, one per lane, and the first four entries of
// this lane's slot (the output columns do not depend on the row max).  The
// row max and the denominator come from the (m, l) pairs by wave-wide
// reductions, then the slots' weighted sums meet by lane shuffles.  On the
// short rows of a decode batch this is about 1 us faster per call than the
// running-max merge, which long rows need.  Out-of-range slots read entry 0
// and get weight 0.
template <class O, int D, bool COMPACT, class Idx>
__device__ inline void merge_short(const ReduceParams& p, int n, Idx idx, size_t row) {
    constexpr int CW = D / 16;                 // columns per lane
    constexpr int SLOTS = 4;                   // entry slots per row
    constexpr int U = 4;                       // entries per slot per round
    typedef float colv __attribute__((ext_vector_type(CW)));
    typedef _Float16 hcol __attribute__((ext_vector_type(CW)));

    const int lane = threadIdx.x & 63;
    const int j = lane >> 4;                   // this lane's slot
    const int c = lane & 15;
    // this lane's columns of entry ie, as sums
    auto entry = [&](size_t ie) {
        if constexpr (COMPACT)
            return widen_entry<CW>(*(const hcol*)((const _Float16*)p.ws_o + ie * D + c * CW), p.ws_l[ie]);
        else
            return *(const colv*)(p.ws_o + ie * D + c * CW);
    };

    const size_t i0 = lane < n ? idx(lane) : 0;
    const float m0 = lane < n ? p.ws_m[i0] : -INFINITY;
    const float l0 = lane < n ? p.ws_l[i0] : 0.0f;
    colv o[U];
    float mo[U];
#pragma unroll
    for (int u = 0; u < U; u++) {
        const int e = j + u * SLOTS;
        const size_t ie = idx(e < n ? e : 0);
        o[u] = entry(ie);
        mo[u] = p.ws_m[ie];
    }

    // M and the denominator over all entries (lanes stride by 64).
    float M = m0;
    for (int e = lane + 64; e < n; e += 64) M = fmaxf(M, p.ws_m[idx(e)]);
    M = group_max<64>(M);
    const float Ml = M == -INFINITY ? 0.0f : M * kLog2e;
    float den = lane < n ? exp2f(fmaf(m0, kLog2e, -Ml)) * l0 : 0.0f;
    for (int e = lane + 64; e < n; e += 64) {
        const size_t ie = idx(e);
        den += exp2f(fmaf(p.ws_m[ie], kLog2e, -Ml)) * p.ws_l[ie];
    }
    den = group_sum<64>(den);

    // Weighted sum of this lane's slot, U entries per round.
    colv acc = colv{};
    for (int e0 = j; e0 < n; e0 += SLOTS * U) {
        if (e0 != j) {
#pragma unroll
            for (int u = 0; u < U; u++) {
                const int e = e0 + u * SLOTS;
                const size_t ie = idx(e < n ? e : 0);
                o[u] = entry(ie);
                mo[u] = p.ws_m[ie];
            }
        }
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int e = e0 + u * SLOTS;
            const float w = e < n ? exp2f(fmaf(mo[u], kLog2e, -Ml)) : 0.0f;
#pragma unroll
            for (int q = 0; q < CW; q++) acc[q] = fmaf(w, o[u][q], acc[q]);
        }
    }
    // the four slots of the wave (lanes c, c+16, c+32, c+48)
#pragma unroll
    for (int q = 0; q < CW; q++) acc[q] = strided_sum<16>(acc[q]);
    if (j != 0) return;
    const float inv = den > 0.0f ? 1.0f / den : 0.0f;
    typedef typename O::T OT;
    typedef OT ovec __attribute__((ext_vector_type(CW)));
    ovec r;
#pragma unroll
    for (int q = 0; q < CW; q++) r[q] = O::narrow(acc[q] * inv);
    *(ovec*)((OT*)p.out + row * D + c * CW) = r;
}

// One of the two merges, by the waves a row has.
template <class O, int D, int WPR, bool COMPACT, class Idx>
__device__ inline void merge(const ReduceParams& p, int n, Idx idx, size_t row, int sub) {
    if constexpr (WPR == 1) merge_short<O, D, COMPACT>(p, n, idx, row);
    else merge_row<O, D, WPR, COMPACT>(p, n, idx, row, sub);
}

// ---- fixed partitions -------------------------------------------------------

template <class O, int D, int WPR>
__global__ __launch_bounds__(64 * wg_waves(WPR)) __attribute__((amdgpu_waves_per_eu(waves_per_simd(WPR))))
void reduce_kernel(ReduceParams p) {
    constexpr int RPB = wg_waves(WPR) / WPR;   // rows per workgroup
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
    merge<O, D, WPR, false>(p, nparts, [&](int k) { return base + (size_t)k; }, (size_t)row, sub);
}

// ---- balanced split ---------------------------------------------------------

// Rows of a balanced call: the grid is (groups of RPB query heads, sequence,
// query token), so a row's place needs no division.  The decode wrote, per
// (sequence, KV head) stream, its first and last chunk (and the slot of its
// piece in the first): entry e of the row is slot 0 or 1 of chunk c0 + e.
// MULTI: rows of a multi-query call, (sequence s, query token j <
// max_query_len of it, head); the output row is (query_start[s] + j, head),
// a token's column in its stream is j * G + head % G, and a token placed
// before its sequence (its column saw nothing) gets a zero row.
template <class O, int D, int WPR, bool MULTI>
__global__ __launch_bounds__(64 * wg_waves(WPR)) __attribute__((amdgpu_waves_per_eu(waves_per_simd(WPR))))
void reduce_balanced_kernel(ReduceParams p) {
    constexpr int RPB = wg_waves(WPR) / WPR;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int sub = wave % WPR;
    const int hq = blockIdx.x * RPB + wave / WPR;
    const int s = blockIdx.y;
    const int j = blockIdx.z;
    const int32_t* hdr = p.ws_hdr;
    if ((blockIdx.x | blockIdx.y | blockIdx.z) == 0 && threadIdx.x == 0) {
        // The decode kernel is done with the chunk counter: return it to 0,
        // below any call's base, so that the next call takes it over even
        // when it carries the same call number (a replayed graph freezes
        // the number in the kernel's arguments).
        *(unsigned long long*)(const_cast<int32_t*>(hdr) + kHdrCounter) = 0ull;
    }
    if (hq >= p.Hq) return;
    const int S = MULTI ? p.S_seq : p.S;
    const int h = p.g_shift >= 0 ? hq >> p.g_shift : hq / p.G;
    const int gh = hq - h * p.G;                // head within the group
    // Every word the row needs is loaded before any of them is tested: the
    // header, the sequence's prefix entries, the stream's chunk range and,
    // for MULTI, its query range and length.  All of them lie inside the
    // workspace and the arrays the call passed.
    const int magic = hdr[kHdrMagic];
    const int nW = hdr[kHdrNW];
    const int Hkv = hdr[kHdrHkv];
    const int G = hdr[kHdrG];
    const int chunks = hdr[kHdrChunks];
    const int p0 = p.ws_pre[s], p1 = p.ws_pre[s + 1];
    const int32_t* rng = p.ws_pre + S + 1 + 2 * (s * p.Hkv + h);
    const int r0 = rng[0], r1 = rng[1];
    const int q0 = MULTI ? p.q_start[s] : 0;
    const int q1 = MULTI ? p.q_start[s + 1] : 0;
    const int Lraw = MULTI ? p.lens[s] : 0;
    // A workspace not written by a balanced call of this shape (or inputs
    // breaking the call's contract): write nothing rather than follow its
    // indices.  One condition of every word, combined without short cuts, so
    // that no load is deferred behind a test of another.
    const int c0 = r0 & 0x7FFFFFFF, c1 = r1;
    const bool bad = (magic != kBalancedMagic) | (nW < 1) | (nW > kBalancedMaxWaves) |
                     (G != p.G) | (Hkv != p.Hkv) | (chunks < 0) |
                     ((int64_t)chunks > max_chunks(nW)) | (p1 < p0) |
                     (MULTI & ((q1 < q0) | (Lraw < 0)));
    if (bad) return;
    int col = gh, ncol = G;
    size_t orow = (size_t)s * p.Hq + hq;        // output row
    typedef typename O::T OT;
    auto zero_row = [&]() {
        if (sub == 0)
            for (int d = lane; d < D; d += 64) ((OT*)p.out)[orow * D + d] = O::narrow(0.0f);
    };
    if constexpr (MULTI) {
        const int QPG = 16 / G;
        const int n = min(q1 - q0, QPG);
        if (j >= n) return;                     // no such query token
        orow = (size_t)(q0 + j) * p.Hq + hq;
        col = j * G + gh;
        ncol = QPG * G;
        const int L = Lraw < p.len_cap ? Lraw : p.len_cap;
        if (L - n + j < 0) {                    // its column saw no token
            zero_row();
            return;
        }
    }
    if (p1 == p0) {                             // no tokens: a zero row
        zero_row();
        return;
    }
    if (c0 == c1) return;                       // one chunk held it: decode wrote the row
    if (c1 < c0 || c1 >= chunks) return;        // not ranges of this call
    const int slot0 = (int)((uint32_t)r0 >> 31);
    merge<O, D, WPR, MULTI>(
        p, c1 - c0 + 1,
        [&](int e) {
            const int slot = e == 0 ? slot0 : 0;
            return ((size_t)(c0 + e) * 2 + slot) * ncol + col;
        },
        orow, sub);
}

// Balanced rows of many streams: a wave serves four columns of one
// (sequence, KV head) stream, one row each (16 lanes, D / 16 output values
// per lane), so the header, the stream's chunk range and, for MULTI, its
// query range are read once per four rows, and a stream whose rows the
// decode finished costs one wave per four rows.  The grid is (groups of
// four such waves, sequence); a stream has ceil(ncol / 4) waves.  Entries
// are merged four per round with the running-max update of merge_row.
template <class O, int D, bool MULTI>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(8)))
void reduce_group_kernel(ReduceParams p) {
    constexpr int CW = D / 16;                  // output values per lane
    constexpr int U = 4;                        // entries per round
    typedef float colv __attribute__((ext_vector_type(CW)));
    typedef _Float16 hcol __attribute__((ext_vector_type(CW)));
    const int lane = threadIdx.x & 63;
    const int s = blockIdx.y;
    const int32_t* hdr = p.ws_hdr;
    if ((blockIdx.x | blockIdx.y) == 0 && threadIdx.x == 0) {
        // the decode kernel is done with the chunk counter (as in
        // reduce_balanced_kernel)
        *(unsigned long long*)(const_cast<int32_t*>(hdr) + kHdrCounter) = 0ull;
    }
    const int ncol = MULTI ? 16 : p.G;          // columns (rows) per stream
    const int wps = (ncol + 3) >> 2;            // waves per stream
    const int u = blockIdx.x * kWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (u >= p.Hkv * wps) return;
    const int h = u / wps;
    const int c = (u - h * wps) * 4 + (lane >> 4);   // this lane's column
    const int S = MULTI ? p.S_seq : p.S;
    // every word first, then the tests (see reduce_balanced_kernel)
    const int magic = hdr[kHdrMagic];
    const int nW = hdr[kHdrNW];
    const int Hkv = hdr[kHdrHkv];
    const int G = hdr[kHdrG];
    const int chunks = hdr[kHdrChunks];
    const int p0 = p.ws_pre[s], p1 = p.ws_pre[s + 1];
    const int32_t* rng = p.ws_pre + S + 1 + 2 * (s * p.Hkv + h);
    const int r0 = rng[0], r1 = rng[1];
    const int q0 = MULTI ? p.q_start[s] : 0;
    const int q1 = MULTI ? p.q_start[s + 1] : 0;
    const int Lraw = MULTI ? p.lens[s] : 0;
    const int c0 = r0 & 0x7FFFFFFF, c1 = r1;
    const bool bad = (magic != kBalancedMagic) | (nW < 1) | (nW > kBalancedMaxWaves) |
                     (G != p.G) | (Hkv != p.Hkv) | (chunks < 0) |
                     ((int64_t)chunks > max_chunks(nW)) | (p1 < p0) |
                     (MULTI & ((q1 < q0) | (Lraw < 0)));
    if (bad) return;
    // the lane's row: whether it exists, saw any token, and where it goes
    bool live = c < ncol, blind = false;
    size_t orow = (size_t)s * p.Hq + (size_t)h * G + (size_t)c;
    if constexpr (MULTI) {
        const int j = c / G;                    // query token of the column
        const int n = min(q1 - q0, 16 / G);
        const int L = Lraw < p.len_cap ? Lraw : p.len_cap;
        live = live && j < n;
        blind = L - n + j < 0;
        orow = (size_t)(q0 + j) * p.Hq + (size_t)h * G + (size_t)(c % G);
    }
    typedef typename O::T OT;
    typedef OT ovec __attribute__((ext_vector_type(CW)));
    const int c16 = lane & 15;
    auto put = [&](const colv& v, float scale) {
        if (!live) return;
        ovec r;
#pragma unroll
        for (int q = 0; q < CW; q++) r[q] = O::narrow(v[q] * scale);
        *(ovec*)((OT*)p.out + orow * D + c16 * CW) = r;
    };
    colv acc = colv{};
    if (p1 == p0) {                             // no tokens: zero rows
        put(acc, 0.0f);
        return;
    }
    if (c0 == c1) {                             // one chunk held it: decode wrote the rows
        if (MULTI && blind) put(acc, 0.0f);
        return;
    }
    if (c1 < c0 || c1 >= chunks) return;        // not ranges of this call
    const int slot0 = (int)((uint32_t)r0 >> 31);
    const int cc = c < ncol ? c : ncol - 1;     // idle lanes read a live column
    const int n_e = c1 - c0 + 1;
    float m_run = -INFINITY, l_run = 0.0f;      // reference max (log2 units), sum
    for (int e0 = 0; e0 < n_e; e0 += U) {
        colv o[U];
        hcol hv[U];
        float m[U], l[U];
#pragma unroll
        for (int k = 0; k < U; k++) {          // the round's loads, all at once
            const int e = e0 + k < n_e ? e0 + k : n_e - 1;
            const size_t ie = ((size_t)(c0 + e) * 2 + (e == 0 ? slot0 : 0)) * ncol + cc;
            if constexpr (MULTI) hv[k] = *(const hcol*)((const _Float16*)p.ws_o + ie * D + c16 * CW);
            else o[k] = *(const colv*)(p.ws_o + ie * D + c16 * CW);
            m[k] = p.ws_m[ie];
            l[k] = p.ws_l[ie];
        }
        __builtin_amdgcn_sched_barrier(0);
        float bm = m_run;
#pragma unroll
        for (int k = 0; k < U; k++) {
            m[k] = e0 + k < n_e ? m[k] * kLog2e : -INFINITY;   // repeats carry no weight
            bm = fmaxf(bm, m[k]);
        }
        const float ref = bm == -INFINITY ? 0.0f : bm;
        const float f = exp2f(m_run - ref);
        l_run *= f;
        acc *= f;
#pragma unroll
        for (int k = 0; k < U; k++) {
            const float w = exp2f(m[k] - ref);
            l_run = fmaf(w, l[k], l_run);
            if constexpr (MULTI) {              // compact entries: sums = x 2^(e-15) l
                const float f = w * compact_scale(l[k]);
#pragma unroll
                for (int q = 0; q < CW; q++) acc[q] = fmaf(f, (float)hv[k][q], acc[q]);
            } else {
#pragma unroll
                for (int q = 0; q < CW; q++) acc[q] = fmaf(w, o[k][q], acc[q]);
            }
        }
        m_run = bm;
    }
    put(acc, l_run > 0.0f && !blind ? 1.0f / l_run : 0.0f);
}

template <class O, int D, int WPR, bool BAL>
hipError_t launch_r(const ReduceParams& p, hipStream_t st) {
    constexpr int RPB = wg_waves(WPR) / WPR;
    const dim3 block(64 * wg_waves(WPR));
    if (BAL) {
        // (groups of query heads, sequences, query tokens per sequence)
        const int seqs = p.q_start ? p.S_seq : p.S;
        const dim3 grid((unsigned)((p.Hq + RPB - 1) / RPB), (unsigned)seqs,
                        (unsigned)(p.q_start ? p.S / p.S_seq : 1));
        if (p.q_start)
            return launch_kernel(reduce_balanced_kernel<O, D, WPR, true>, grid, block, st, p);
        return launch_kernel(reduce_balanced_kernel<O, D, WPR, false>, grid, block, st, p);
    }
    const long rows = (long)p.S * p.Hq;
    const dim3 grid((unsigned)((rows + RPB - 1) / RPB));
    return launch_kernel(reduce_kernel<O, D, WPR>, grid, block, st, p);
}

template <class O, int D, bool BAL>
hipError_t launch_w(const ReduceParams& p, int wpr, hipStream_t st) {
    if (wpr >= 8) return launch_r<O, D, 8, BAL>(p, st);
    if (wpr >= 4) return launch_r<O, D, 4, BAL>(p, st);
    return launch_r<O, D, 1, BAL>(p, st);
}

template <class O, bool BAL>
hipError_t launch_d(const ReduceParams& p, int wpr, hipStream_t st) {
    if (p.D == 64) return launch_w<O, 64, BAL>(p, wpr, st);
    if (p.D == 128) return launch_w<O, 128, BAL>(p, wpr, st);
    return hipErrorInvalidValue;
}

template <bool BAL>
hipError_t launch_o(int out_dt, const ReduceParams& p, int wpr, hipStream_t st) {
    switch (out_dt) {
    case kF32: return launch_d<F32, BAL>(p, wpr, st);
    case kF16: return launch_d<F16, BAL>(p, wpr, st);
    case kBF16: return launch_d<BF16, BAL>(p, wpr, st);
    default: return hipErrorInvalidValue;
    }
}

template <class O, int D>
hipError_t launch_group_d(const ReduceParams& p, hipStream_t st) {
    const int ncol = p.q_start ? 16 : p.G;
    const long waves = (long)p.Hkv * ((ncol + 3) / 4);
    const dim3 grid((unsigned)((waves + kWaves - 1) / kWaves),
                    (unsigned)(p.q_start ? p.S_seq : p.S)),
        block(64 * kWaves);
    if (p.q_start) return launch_kernel(reduce_group_kernel<O, D, true>, grid, block, st, p);
    return launch_kernel(reduce_group_kernel<O, D, false>, grid, block, st, p);
}

template <class O>
hipError_t launch_group_o(const ReduceParams& p, hipStream_t st) {
    if (p.D == 64) return launch_group_d<O, 64>(p, st);
    if (p.D == 128) return launch_group_d<O, 128>(p, st);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_reduce(int out_dt, const ReduceParams& p, hipStream_t st) {
    // waves per row by the most partitions a row can have
    return launch_o<false>(out_dt, p, p.P_max > 128 ? 8 : (p.P_max > 32 ? 4 : 1), st);
}

hipError_t launch_reduce_balanced(int out_dt, const ReduceParams& p, hipStream_t st) {
    // Few rows (long contexts, each row split over many chunks): eight
    // waves per row.  Many decode rows: one wave per row (on the ragged GQA
    // batch 4.95 us against 7.3 us at four rows per wave, whose fewer waves
    // hide less latency).  Many multi-query rows (16 per stream): four rows
    // of one stream per wave (9.4 us against 12.2 us at one per row).
    if ((long)p.S * p.Hq <= 2048) return launch_o<true>(out_dt, p, 8, st);
    if (!p.q_start) return launch_o<true>(out_dt, p, 1, st);
    switch (out_dt) {
    case kF32: return launch_group_o<F32>(p, st);
    case kF16: return launch_group_o<F16>(p, st);
    case kBF16: return launch_group_o<BF16>(p, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace pkv
