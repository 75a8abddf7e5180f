// multi_query.hip - paged attention for several new query tokens per
// sequence: chunked prefill ("vLLM 推理引擎源码级拆解" §6.3: a long prompt's
// prefill cut into chunks run between decode steps) and speculative
// verification (§6.5: the large model checks several drafted tokens in one
// pass).  The Qn new tokens of sequence s are its last Qn cached tokens
// (already stored by reshape_and_cache); query token i sits at position
// L - Qn + i and attends to tokens 0 .. L - Qn + i through the block table,
// with the same single-pass online softmax as decode.
//
// Work layout.  The matrix-core tile of tile_mfma.hpp takes 16 B columns;
// here a column is a (query token, query head) pair: column c holds head
// c % G of query token c / G, so a wavefront serves 16 / G consecutive query
// tokens of one sequence and all G heads of one KV head, and each K/V tile it
// loads feeds every one of them.  Column c drops the tokens past its own
// position (the causal limit inside the chunk).  A wavefront reads tokens
// 0 .. (its last query token's position) with the decode kernel's pipeline:
// windows of 64 table entries, a ring of DEPTH tiles in flight, K tiles
// staged in LDS in row order (TileMath; on MI355X verification at P = 512
// went from 364 to 332 µs per call).  Units are
// numbered with the query group innermost, so the wavefronts that re-read
// one sequence's K/V for its different groups run side by side and share it
// through the caches.
//
// Split-K (partition_size P > 0), for long contexts and short drafts: the
// units are (sequence, partition, KV head, query group) in the decode
// kernel's order (full partitions first, split_units.hpp), a unit reads the
// tokens of its partition, and each column's row is written directly when
// the column sees at most P tokens (partition 0 holds them all) or left as
// partials otherwise.  The call then runs the decode reduce over the rows
// (query token, head), with the number of tokens each query token sees
// written by this kernel into the workspace.
#include "split_units.hpp"
#include "tile_mfma.hpp"

namespace pkv {
namespace {

using namespace mfma;

constexpr int kWaves = 4;

// KLDS: K tiles staged in LDS, DEPTH slots per wave (TileMath); the ring
// waits for slot j with an explicit count, as in decode_mfma_kernel.
template <class Q, class C, int D, bool PAIR, int DEPTH, bool SPLIT, bool KLDS>
__global__ __launch_bounds__(64 * kWaves) void multi_query_kernel(DecodeParams p) {
    typedef TileMath<Q, C, D, PAIR, KLDS> TM;
    extern __shared__ __attribute__((aligned(16))) char lds_k[];
    typedef typename TM::T T;
    typedef typename TM::v8 v8;
    const TM tm;
    const int lane = tm.lane;

    const int unit = blockIdx.x * kWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int cg = unit % p.max_groups;
    const int h = (unit / p.max_groups) % p.Hkv;
    int s = unit / p.max_groups / p.Hkv, part = 0;
    if constexpr (SPLIT) {
        if (unit == 0) {
            // the reduce reads ws_len for num_seqs * max_query_len rows: rows
            // past the batch's query tokens see nothing
            for (int i = p.q_start[p.S] + lane; i < p.len_rows; i += 64) p.ws_len[i] = 0;
        }
        if (!find_unit(p, s, &s, &part)) return;
        s = __builtin_amdgcn_readfirstlane(s);
        part = __builtin_amdgcn_readfirstlane(part);
    } else if (s >= p.S) {
        return;
    }
    const int G = p.G;
    const int QPG = 16 / G;                            // query tokens per wavefront
    const int q0 = __builtin_amdgcn_readfirstlane(p.q_start[s]);
    const int Qn = __builtin_amdgcn_readfirstlane(p.q_start[s + 1]) - q0;
    const int qbase = cg * QPG;
    if (qbase >= Qn) return;
    const int nq = min(QPG, Qn - qbase);
    const int ncols = nq * G;
    // split rows live in a workspace of num_seqs * max_query_len query
    // tokens: a batch that breaks Qn <= max_query_len loses its later rows
    // rather than write past it
    if (SPLIT && q0 + qbase + nq > p.len_rows) return;
    int L = __builtin_amdgcn_readfirstlane(p.lens[s]);
    L = L < p.len_cap ? L : p.len_cap;
    const int pos0 = L - Qn + qbase;                   // position of the group's first token
    const int t_end = pos0 + nq;                       // tokens [0, t_end) are seen
    if constexpr (SPLIT) {
        if (part == 0 && h == 0 && lane < nq) p.ws_len[q0 + qbase + lane] = max(pos0 + lane + 1, 0);
    }
    const int t_begin = SPLIT ? part * p.P : 0;
    const int t_stop = SPLIT ? min(t_end, t_begin + p.P) : t_end;   // this unit's tokens

    auto out_row = [&](int c) {
        return (T*)p.out + ((size_t)(q0 + qbase + c / G) * p.Hq + (size_t)h * G + c % G) * D;
    };
    if (t_end <= 0) {                                  // every token of the group precedes the sequence
        if (part == 0)
            for (int c = 0; c < ncols; c++)
                for (int i = lane; i < D; i += 64) out_row(c)[i] = (T)0.0f;
        return;
    }
    if (t_begin >= t_stop) return;                     // no token of the group in this partition

    // B operand: column j16 = (token j16 / G, head j16 % G); zero past ncols
    v8 qb[TM::KS];
    {
        const T* qrow = (const T*)p.q +
                        ((size_t)(q0 + qbase + tm.j16 / G) * p.Hq + (size_t)h * G + tm.j16 % G) * D;
#pragma unroll
        for (int kk = 0; kk < TM::KS; kk++) {
            const int d0 = TM::kFp8 ? (kk >> 1) * 64 + 16 * tm.g4 + (kk & 1) * 8 : 32 * kk + 8 * tm.g4;
            qb[kk] = tm.j16 < ncols ? *(const v8*)(qrow + d0) : v8{};
        }
    }
    // this lane's column: last token it may see (-1: none)
    const int pc = tm.j16 < ncols ? pos0 + tm.j16 / G : -1;

    const Head hd = make_head<C, D>(p, h);
    const int32_t* table = p.tables + (size_t)s * p.max_blocks;
    const int nblk = (t_stop + p.bs - 1) >> hd.bs_shift;

    typename TM::Acc acc;
    tm.reset(acc);
    lds_t* const kring =
        (lds_t*)lds_k + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) * DEPTH * TM::kKSlot;
    auto kslot = [&](int j) { return kring + j * TM::kKSlot; };
    const int wtok = 64 << hd.bs_shift;
    for (int w0 = t_begin; w0 < t_stop; w0 += wtok) {
        const int w1 = min(t_stop, w0 + wtok);
        const int wb = w0 >> hd.bs_shift;
        const int win = (wb + lane < nblk) ? table[wb + lane] : 0;
        typename TM::Tile tl[DEPTH];
#pragma unroll
        for (int j = 0; j < DEPTH; j++) {
            tm.issue(hd, w0 + 16 * j, w1 - 1 - (w0 + 16 * j), wb, win, tl[j], kslot(j));
            if constexpr (KLDS) __builtin_amdgcn_sched_barrier(0);
        }
        for (int t0 = w0; t0 < w1; t0 += 16 * DEPTH) {
#pragma unroll
            for (int j = 0; j < DEPTH; j++) {
                const int tj = t0 + 16 * j;
                if constexpr (KLDS) {
                    vm_wait<(DEPTH - 1) * TM::kLoadsPerTile>();
                    __builtin_amdgcn_sched_barrier(0);
                }
                if (j == 0 || tj < w1)
                    tm.template consume<true>(acc, qb, p.scale_log2, t_stop - 1 - tj, tl[j], pc - tj,
                                              kslot(j));
                if constexpr (KLDS) __builtin_amdgcn_sched_barrier(0);
                const int tn = tj + 16 * DEPTH;
                tm.issue(hd, tn, w1 - 1 - tn, wb, win, tl[j], kslot(j));
                if constexpr (KLDS) __builtin_amdgcn_sched_barrier(0);
            }
        }
    }

    // row of column c in the reduce's layout: (query token, query head)
    auto row_of = [&](int c) {
        return (size_t)(q0 + qbase + c / G) * p.Hq + (size_t)h * G + c % G;
    };
    tm.finish_each(
        acc, ncols,
        [&](int c) { return !SPLIT || (part == 0 && pos0 + c / G + 1 <= p.P); }, p.v_scale,
        out_row, [&](int c) { return p.ws_m + row_of(c) * p.P_max + part; },
        [&](int c) { return p.ws_l + row_of(c) * p.P_max + part; },
        [&](int c) { return p.ws_o + (row_of(c) * p.P_max + part) * D; });
    // the ring's last round may still be landing in the K slots
    if constexpr (KLDS) vm_wait<0>();
}

// Long query runs (chunked prefill): every wavefront of the kernel above
// reads the sequence's K/V for its 16 / G tokens, so a 512-token chunk reads
// it 128 times (from the caches after the first).  Here a wavefront carries
// NB column blocks (NB * 16 / G consecutive query tokens, each block with
// its own query operand, causal limits and accumulators) and feeds every K/V
// tile it loads to all of them: NB times the arithmetic per byte loaded.
// One pass (no split); one wavefront per SIMD, the accumulators and ring
// spilling into the accumulation registers.
template <class Q, class C, int D, bool PAIR, int DEPTH, int NB, bool KLDS>
__global__ __launch_bounds__(64 * kWaves, 1) void multi_query_wide_kernel(DecodeParams p) {
    typedef TileMath<Q, C, D, PAIR, KLDS> TM;
    extern __shared__ __attribute__((aligned(16))) char lds_k[];
    typedef typename TM::T T;
    typedef typename TM::v8 v8;
    const TM tm;
    const int lane = tm.lane;

    const int unit = blockIdx.x * kWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int cg = unit % p.max_groups;
    const int h = (unit / p.max_groups) % p.Hkv;
    const int s = unit / p.max_groups / p.Hkv;
    if (s >= p.S) return;
    const int G = p.G;
    const int QPG = 16 / G;                            // query tokens per column block
    const int q0 = __builtin_amdgcn_readfirstlane(p.q_start[s]);
    const int Qn = __builtin_amdgcn_readfirstlane(p.q_start[s + 1]) - q0;
    const int qbase = cg * QPG * NB;                   // the wave's first query token
    if (qbase >= Qn) return;
    int L = __builtin_amdgcn_readfirstlane(p.lens[s]);
    L = L < p.len_cap ? L : p.len_cap;
    const int nq = min(QPG * NB, Qn - qbase);          // query tokens of this wave
    const int t_end = L - Qn + qbase + nq;             // tokens the last one sees

    // row of column c of block b
    auto out_row = [&](int b, int c) {
        return (T*)p.out +
               ((size_t)(q0 + qbase + b * QPG + c / G) * p.Hq + (size_t)h * G + c % G) * D;
    };
    if (t_end <= 0) {                                  // every token precedes the sequence
        for (int c = 0; c < nq * G; c++)
            for (int i = lane; i < D; i += 64) out_row(0, c)[i] = (T)0.0f;
        return;
    }

    v8 qb[NB][TM::KS];
    int pc[NB];                                        // this lane's column: last token seen
    int ncols[NB];
#pragma unroll
    for (int b = 0; b < NB; b++) {
        const int tb = qbase + b * QPG;
        const int nqb = max(0, min(QPG, Qn - tb));
        ncols[b] = nqb * G;
        const T* qrow = (const T*)p.q +
                        ((size_t)(q0 + tb + tm.j16 / G) * p.Hq + (size_t)h * G + tm.j16 % G) * D;
#pragma unroll
        for (int kk = 0; kk < TM::KS; kk++) {
            const int d0 = TM::kFp8 ? (kk >> 1) * 64 + 16 * tm.g4 + (kk & 1) * 8 : 32 * kk + 8 * tm.g4;
            qb[b][kk] = tm.j16 < ncols[b] ? *(const v8*)(qrow + d0) : v8{};
        }
        pc[b] = tm.j16 < ncols[b] ? L - Qn + tb + tm.j16 / G : -1;
    }

    const Head hd = make_head<C, D>(p, h);
    const int32_t* table = p.tables + (size_t)s * p.max_blocks;
    const int nblk = (t_end + p.bs - 1) >> hd.bs_shift;
    typename TM::Acc acc[NB];
#pragma unroll
    for (int b = 0; b < NB; b++) tm.reset(acc[b]);
    lds_t* const kring =
        (lds_t*)lds_k + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) * DEPTH * TM::kKSlot;
    auto kslot = [&](int j) { return kring + j * TM::kKSlot; };
    const int wtok = 64 << hd.bs_shift;
    for (int w0 = 0; w0 < t_end; w0 += wtok) {
        const int w1 = min(t_end, w0 + wtok);
        const int wb = w0 >> hd.bs_shift;
        const int win = (wb + lane < nblk) ? table[wb + lane] : 0;
        typename TM::Tile tl[DEPTH];
#pragma unroll
        for (int j = 0; j < DEPTH; j++) {
            tm.issue(hd, w0 + 16 * j, w1 - 1 - (w0 + 16 * j), wb, win, tl[j], kslot(j));
            if constexpr (KLDS) __builtin_amdgcn_sched_barrier(0);
        }
        for (int t0 = w0; t0 < w1; t0 += 16 * DEPTH) {
#pragma unroll
            for (int j = 0; j < DEPTH; j++) {
                const int tj = t0 + 16 * j;
                if constexpr (KLDS) {
                    vm_wait<(DEPTH - 1) * TM::kLoadsPerTile>();
                    __builtin_amdgcn_sched_barrier(0);
                }
                if (j == 0 || tj < w1) {
#pragma unroll
                    for (int b = NB - 1; b >= 0; b--)
                        tm.template consume<true>(acc[b], qb[b], p.scale_log2, t_end - 1 - tj,
                                                  tl[j], pc[b] - tj, kslot(j));
                }
                if constexpr (KLDS) __builtin_amdgcn_sched_barrier(0);
                const int tn = tj + 16 * DEPTH;
                tm.issue(hd, tn, w1 - 1 - tn, wb, win, tl[j], kslot(j));
                if constexpr (KLDS) __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
#pragma unroll
    for (int b = 0; b < NB; b++)
        tm.finish_each(
            acc[b], ncols[b], [&](int) { return true; }, p.v_scale,
            [&](int c) { return out_row(b, c); }, [&](int) { return (float*)nullptr; },
            [&](int) { return (float*)nullptr; }, [&](int) { return (float*)nullptr; });
    // the ring's last round may still be landing in the K slots
    if constexpr (KLDS) vm_wait<0>();
}

// Tiles in flight per wavefront, as in the one-pass decode kernel.
template <bool PAIR>
constexpr int pipeline_depth() {
    return PAIR ? 2 : 4;
}

// K tiles go through LDS (DEPTH slots per wave), 8-token blocks included
// where each row-order load covers one block's rows (at most 8 rows a load).
template <class Q, class C, int D, bool PAIR>
constexpr bool k_in_lds() {
    return !PAIR || 1024 / (D * C::kBytes) <= 8;
}
template <class Q, class C, int D, bool PAIR>
constexpr size_t k_ring_bytes() {
    return (size_t)kWaves * pipeline_depth<PAIR>() * TileMath<Q, C, D, false, true>::kKSlot;
}

template <class Q, class C, int D, int NB, bool PAIR>
hipError_t launch_wide_p(const DecodeParams& p, dim3 grid, dim3 block, hipStream_t st) {
    constexpr bool L = k_in_lds<Q, C, D, PAIR>();
    void* args[] = {const_cast<DecodeParams*>(&p)};
    return hipLaunchKernel(
        reinterpret_cast<const void*>(multi_query_wide_kernel<Q, C, D, PAIR, pipeline_depth<PAIR>(), NB, L>),
        grid, block, args, L ? k_ring_bytes<Q, C, D, PAIR>() : 0, st);
}

template <class Q, class C, int D, int NB>
hipError_t launch_wide(const DecodeParams& p, dim3 grid, dim3 block, hipStream_t st) {
    if (p.bs == 8) return launch_wide_p<Q, C, D, NB, true>(p, grid, block, st);
    return launch_wide_p<Q, C, D, NB, false>(p, grid, block, st);
}

template <class Q, class C, int D, bool SPLIT, bool PAIR>
hipError_t launch_ds_p(const DecodeParams& p, dim3 grid, dim3 block, hipStream_t st) {
    constexpr bool L = k_in_lds<Q, C, D, PAIR>();
    void* args[] = {const_cast<DecodeParams*>(&p)};
    return hipLaunchKernel(
        reinterpret_cast<const void*>(multi_query_kernel<Q, C, D, PAIR, pipeline_depth<PAIR>(), SPLIT, L>),
        grid, block, args, L ? k_ring_bytes<Q, C, D, PAIR>() : 0, st);
}

template <class Q, class C, int D, bool SPLIT>
hipError_t launch_ds(const DecodeParams& p, dim3 grid, dim3 block, hipStream_t st) {
    if (p.bs == 8) return launch_ds_p<Q, C, D, SPLIT, true>(p, grid, block, st);
    return launch_ds_p<Q, C, D, SPLIT, false>(p, grid, block, st);
}

template <class Q, class C, int D>
hipError_t launch_dd(const DecodeParams& p, dim3 grid, dim3 block, hipStream_t st) {
    if (p.P > 0) return launch_ds<Q, C, D, true>(p, grid, block, st);
    if (p.col_blocks == 4) return launch_wide<Q, C, D, 4>(p, grid, block, st);
    if (p.col_blocks == 2) return launch_wide<Q, C, D, 2>(p, grid, block, st);
    return launch_ds<Q, C, D, false>(p, grid, block, st);
}

template <class Q, class C>
hipError_t launch_d(const DecodeParams& p, hipStream_t st) {
    const long units = (long)p.S * p.P_max * p.max_groups * p.Hkv;
    const dim3 grid((unsigned)((units + kWaves - 1) / kWaves)), block(64 * kWaves);
    if (p.D == 64) return launch_dd<Q, C, 64>(p, grid, block, st);
    if (p.D == 128) return launch_dd<Q, C, 128>(p, grid, block, st);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_multi_query(int qdt, int cdt, const DecodeParams& p, hipStream_t st) {
    if (!decode_mfma_supported(qdt, cdt, p.D, p.G)) return hipErrorInvalidValue;
    if (qdt == kBF16) {
        if (cdt == kFP8) return launch_d<BF16, FP8>(p, st);
        return launch_d<BF16, BF16>(p, st);
    }
    if (cdt == kFP8) return launch_d<F16, FP8>(p, st);
    return launch_d<F16, F16>(p, st);
}

}  // namespace pkv
