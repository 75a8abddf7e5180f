// decode_mfma.hip - paged decode attention on the CDNA4 matrix cores, one
// work unit per wavefront (one-pass and fixed-partition split-K modes).
//
// Same contract as the vector-ALU kernel (single query per sequence against
// its block-table-indirect K/V with an online softmax, "vLLM 推理引擎源码级拆解"
// §2.3), for f16/bf16 queries over f16/bf16/E4M3 caches.  A wavefront owns one
// unit = (sequence, partition, KV head) and serves the G <= 16 query heads of
// the GQA group with the matrix-core tile of tile_mfma.hpp.
//
// Pipeline.  Several tiles are in flight per wavefront: the loop is unrolled
// by hand over a ring of tile buffers so that the loads of later tiles are
// issued before a tile is consumed and no register copy forces an early
// wait.  The unit is walked in windows of 64 block-table entries.
//
// Split-K work list.  With partition_size P > 0, sequence s contributes
// max(1, ceil(L_s / P)) partitions.  The (sequence, partition) pairs are
// numbered without gaps, every full-length partition first and the last,
// ragged partition of each sequence after them, so every wavefront of the
// grid that has work owns a whole unit of at most P tokens and the short
// units fill the tail of the grid; waves numbered past the total exit at
// once.  Each wave finds its pair from the lengths with a wavefront prefix
// sum.
#include "split_units.hpp"
#include "tile_mfma.hpp"

namespace pkv {
namespace {

using namespace mfma;

constexpr int kWaves = 4;

// head_dim of a tile math type
template <class TM>
__device__ constexpr int D_of() { return TM::NT * 16; }

// Walks tokens [t_begin, t_end) of one unit: DEPTH tiles in flight in a ring
// of tile buffers unrolled by hand.  Tile j of each round is consumed, then
// refilled with the tile DEPTH positions ahead, so DEPTH - 1 tiles stay in
// flight during the arithmetic; loads are issued unconditionally (dead tiles
// read zeros).  The unit is walked in windows of 64 table entries (one per
// lane); a split-K partition of at most 64 blocks is a single window.  PR:
// 8-token blocks (a tile spans two).  KLDS: TM stages K tiles in LDS, slot j
// of the ring at kring + j * TM::kKSlot; the loads carry no register to wait
// on, so slot j is read once at most the loads of the DEPTH - 1 tiles issued
// after it are in flight (every round issues all DEPTH tiles in ring order,
// dead ones included; scheduling barriers keep whole tiles in that order).
template <bool PR, int DEPTH, bool KLDS = false, class TM>
__device__ inline void walk_unit(const TM& tm, const Head& hd, const int32_t* table,
                                 int t_begin, int t_end, const typename TM::v8 (&qb)[TM::KS],
                                 float scale_log2, typename TM::Acc& acc,
                                 lds_t* kring = nullptr) {
    const int lane = tm.lane;
    const int nblk = (t_end + (1 << hd.bs_shift) - 1) >> hd.bs_shift;   // table entries used
    const int wtok = 64 << hd.bs_shift;
    for (int w0 = t_begin; w0 < t_end; w0 += wtok) {
        const int w1 = min(t_end, w0 + wtok);
        const int wb = w0 >> hd.bs_shift;
        const int win = (wb + lane < nblk) ? table[wb + lane] : 0;
        typename TM::Tile tl[DEPTH];
#pragma unroll
        for (int j = 0; j < DEPTH; j++) {
            tm.template issue_as<PR>(hd, w0 + 16 * j, w1 - 1 - (w0 + 16 * j), wb, win, tl[j],
                                     kring + j * TM::kKSlot);
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
                    tm.consume(acc, qb, scale_log2, t_end - 1 - tj, tl[j], 0, kring + j * TM::kKSlot);
                if constexpr (KLDS) __builtin_amdgcn_sched_barrier(0);
                const int tn = tj + 16 * DEPTH;
                tm.template issue_as<PR>(hd, tn, w1 - 1 - tn, wb, win, tl[j], kring + j * TM::kKSlot);
                if constexpr (KLDS) __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
}

// Selects the unit = (sequence, partition, KV head) of this wavefront; false
// when the wavefront has none.  Everything that selects the unit is
// wave-uniform; readfirstlane tells the compiler so, which keeps block
// descriptors in scalar registers.
__device__ inline bool select_unit(const DecodeParams& p, int* s_out, int* part_out, int* h_out) {
    const int unit = blockIdx.x * kWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    *h_out = unit % p.Hkv;
    const int sp = unit / p.Hkv;
    int s = sp, part = 0;
    if (p.P > 0) {
        if (!find_unit(p, sp, &s, &part)) return false;
        s = __builtin_amdgcn_readfirstlane(s);
        part = __builtin_amdgcn_readfirstlane(part);
    } else if (s >= p.S) {
        return false;
    }
    *s_out = s;
    *part_out = part;
    return true;
}

// DEPTH: tiles whose loads are issued ahead of the arithmetic (the ring).
// KLDS: K tiles staged in LDS (TileMath), DEPTH slots per wave.
template <class Q, class C, int D, bool PAIR, int DEPTH, bool KLDS>
__global__ __launch_bounds__(64 * kWaves) void decode_mfma_kernel(DecodeParams p) {
    typedef TileMath<Q, C, D, PAIR, KLDS> TM;
    extern __shared__ __attribute__((aligned(16))) char lds_k[];
    typedef typename TM::T T;
    const TM tm;
    const int lane = tm.lane;
    int s, part, h;
    if (!select_unit(p, &s, &part, &h)) return;

    const int G = p.G;
    int L = p.lens[s];
    L = L < p.len_cap ? L : p.len_cap;
    T* out = (T*)p.out + ((size_t)s * p.Hq + (size_t)h * G) * D;
    if (L <= 0) {
        for (int i = lane; i < G * D; i += 64) out[i] = (T)0.0f;
        return;
    }
    int t_begin = 0, t_end = L;
    bool final_out = true;
    if (p.P > 0) {
        t_begin = part * p.P;
        t_end = min(L, t_begin + p.P);
        final_out = (L + p.P - 1) / p.P <= 1;
    }

    typename TM::v8 qb[TM::KS];
    tm.load_q((const T*)p.q + ((size_t)s * p.Hq + (size_t)h * G) * D, G, qb);
    const Head hd = make_head<C, D>(p, h);
    typename TM::Acc acc;
    tm.reset(acc);
    lds_t* const kring =
        (lds_t*)lds_k + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) * DEPTH * TM::kKSlot;
    walk_unit<PAIR, DEPTH, KLDS>(tm, hd, p.tables + (size_t)s * p.max_blocks, t_begin, t_end, qb,
                                 p.scale_log2, acc, kring);

    const size_t row0 = (size_t)s * p.Hq + (size_t)h * G;
    tm.finish(
        acc, G, final_out, p.v_scale,
        [&](int head) { return out + (size_t)head * D; },
        [&](int head) { return p.ws_m + (row0 + head) * p.P_max + part; },
        [&](int head) { return p.ws_l + (row0 + head) * p.P_max + part; },
        [&](int head) { return p.ws_o + ((row0 + head) * p.P_max + part) * D; });
    // the ring's last round (dead tiles, zeros) may still be landing in the
    // K slots: let it land before the workgroup's LDS is handed on
    if constexpr (KLDS) vm_wait<0>();
}

// Mixed block sizes ("vLLM 0.5 深度拆解" §1.3: 8, 16 or 32 tokens per
// block, chosen per request).  The pool is kept in pages of p.bs tokens, laid
// out like a pool of p.bs-token blocks; a block of bs_s = seq_bs[s] tokens is
// bs_s / p.bs consecutive pages, and table entries give its first page.  So
// the table is walked in bs_s-token steps, a block's base is (entry * p.bs)
// rows in, and its descriptor covers bs_s rows.  Each wavefront runs the
// 8-token-block loop or the larger-block one for its own sequence.  A block
// size outside [page, 32] is taken as the nearest of the two.  K tiles go
// through LDS as in decode_mfma_kernel (on MI355X the mixed-size batch at
// P = 512 went from 290.9 to 274.5 µs per call).
// One unit of the mixed-size kernel on the tile math TM: 8-token blocks (PR,
// a tile spans two) or larger ones, K staged in LDS when KLDS.
template <bool PR, int DEPTH, bool KLDS, class TM>
__device__ inline void mixed_unit(const TM& tm, const DecodeParams& p, const Head& hd,
                                  const int32_t* table, int s, int h, int part, int t_begin,
                                  int t_end, bool final_out, lds_t* kring) {
    typedef typename TM::T T;
    const int G = p.G;
    T* out = (T*)p.out + ((size_t)s * p.Hq + (size_t)h * G) * D_of<TM>();
    typename TM::v8 qb[TM::KS];
    tm.load_q((const T*)p.q + ((size_t)s * p.Hq + (size_t)h * G) * D_of<TM>(), G, qb);
    typename TM::Acc acc;
    tm.reset(acc);
    walk_unit<PR, DEPTH, KLDS>(tm, hd, table, t_begin, t_end, qb, p.scale_log2, acc, kring);
    const size_t row0 = (size_t)s * p.Hq + (size_t)h * G;
    constexpr int D = D_of<TM>();
    tm.finish(
        acc, G, final_out, p.v_scale,
        [&](int head) { return out + (size_t)head * D; },
        [&](int head) { return p.ws_m + (row0 + head) * p.P_max + part; },
        [&](int head) { return p.ws_l + (row0 + head) * p.P_max + part; },
        [&](int head) { return p.ws_o + ((row0 + head) * p.P_max + part) * D; });
    // the ring's last round may still be landing in the K slots
    if constexpr (KLDS) vm_wait<0>();
}

template <class Q, class C, int D>
__global__ __launch_bounds__(64 * kWaves) void decode_mixed_kernel(DecodeParams p) {
    // 16- and 32-token blocks: K staged in LDS (four slots per wave); 8-token
    // blocks too where each row-order load lies in one block (two slots)
    typedef TileMath<Q, C, D, false, true> TM;
    constexpr bool kPairLds = 1024 / (D * C::kBytes) <= 8;
    typedef TileMath<Q, C, D, true, kPairLds> TM8;
    typedef typename TM::T T;
    extern __shared__ __attribute__((aligned(16))) char lds_k[];
    const int lane = threadIdx.x & 63;
    int s, part, h;
    if (!select_unit(p, &s, &part, &h)) return;

    const int bs_s = __builtin_amdgcn_readfirstlane(p.seq_bs[s]);
    const int shift = bs_s >= 32 ? 5 : max(bs_s >= 16 ? 4 : 3, p.page_shift);
    const int G = p.G;
    int L = p.lens[s];
    L = L < p.len_cap ? L : p.len_cap;
    L = L < (p.max_blocks << shift) ? L : (p.max_blocks << shift);
    if (L <= 0) {
        T* out = (T*)p.out + ((size_t)s * p.Hq + (size_t)h * G) * D;
        for (int i = lane; i < G * D; i += 64) out[i] = (T)0.0f;
        return;
    }
    int t_begin = 0, t_end = L;
    bool final_out = true;
    if (p.P > 0) {
        t_begin = part * p.P;
        t_end = min(L, t_begin + p.P);
        final_out = (L + p.P - 1) / p.P <= 1;
    }

    Head hd = make_head<C, D>(p, h);                  // pages of p.bs tokens
    const uint32_t head_off = (uint32_t)(h * D * C::kBytes);
    hd.bs_shift = shift;
    hd.rec_bytes = (hd.row_bytes << shift) - head_off;
    hd.nb_last = (uint32_t)(p.NB - (1 << (shift - p.page_shift)));
    const int32_t* table = p.tables + (size_t)s * p.max_blocks;
    lds_t* const kring =
        (lds_t*)lds_k + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) * 4 * TM::kKSlot;
    if (shift == 3)
        mixed_unit<true, 2, kPairLds>(TM8(), p, hd, table, s, h, part, t_begin, t_end, final_out,
                                      kring);
    else
        mixed_unit<false, 4, true>(TM(), p, hd, table, s, h, part, t_begin, t_end, final_out,
                                   kring);
}

// Tiles in flight per wavefront.  Four 16-token tiles at head_dim 128 keep
// about 24 KiB of 16-bit K/V in flight per wave at two waves per SIMD; a tile
// spanning two 8-token blocks costs twice the load registers, so that
// variant stays at two.  (Unlike the persistent balanced grid, this grid
// refills a SIMD as its waves finish: one wave per SIMD with a ring of six
// or eight tiles measured 8-10% slower on the ragged GQA batch.)
template <bool PAIR>
constexpr int pipeline_depth() {
    return PAIR ? 2 : 4;
}

// K tiles are staged in LDS (row-order loads, read back in the operand
// layout; see TileMath): kWaves * 4 slots, 64 KiB per workgroup for 16-bit K
// at head_dim 128, so two workgroups share a CU.  8-token blocks (a tile
// spanning two) do the same with two slots per wave where each load covers
// at most 8 rows (all but fp8 at head_dim 64): on MI355X the shared-prefix
// fp8 batch at 8-token blocks went from 67.3 to 56.4 µs per call (rings of
// 3 or 4 tiles read alike).
template <class Q, class C, int D>
hipError_t launch_dd(const DecodeParams& p, dim3 grid, dim3 block, hipStream_t st) {
    void* args[] = {const_cast<DecodeParams*>(&p)};
    if (p.bs == 8) {
        // a two-block tile goes through LDS where each row-order load lies
        // in one block (at most 8 rows per load)
        constexpr int DP = pipeline_depth<true>();
        if constexpr (1024 / (D * C::kBytes) <= 8) {
            constexpr size_t lds = (size_t)kWaves * DP * TileMath<Q, C, D, true, true>::kKSlot;
            return hipLaunchKernel(
                reinterpret_cast<const void*>(decode_mfma_kernel<Q, C, D, true, DP, true>), grid,
                block, args, lds, st);
        }
        return launch_kernel(decode_mfma_kernel<Q, C, D, true, DP, false>, grid, block, st, p);
    }
    constexpr int DP = pipeline_depth<false>();
    constexpr size_t lds = (size_t)kWaves * DP * TileMath<Q, C, D, false, true>::kKSlot;
    return hipLaunchKernel(
        reinterpret_cast<const void*>(decode_mfma_kernel<Q, C, D, false, DP, true>), grid, block,
        args, lds, st);
}

template <class Q, class C>
hipError_t launch_d(const DecodeParams& p, hipStream_t st) {
    const long units = (long)p.S * p.P_max * p.Hkv;
    const dim3 grid((unsigned)((units + kWaves - 1) / kWaves)), block(64 * kWaves);
    if (p.D == 64) return launch_dd<Q, C, 64>(p, grid, block, st);
    if (p.D == 128) return launch_dd<Q, C, 128>(p, grid, block, st);
    return hipErrorInvalidValue;
}

template <class Q, class C>
hipError_t launch_mixed_d(const DecodeParams& p, hipStream_t st) {
    const long units = (long)p.S * p.P_max * p.Hkv;
    const dim3 grid((unsigned)((units + kWaves - 1) / kWaves)), block(64 * kWaves);
    void* args[] = {const_cast<DecodeParams*>(&p)};
    // four K slots per wave (the ring of 16- and 32-token blocks)
    if (p.D == 64)
        return hipLaunchKernel(reinterpret_cast<const void*>(decode_mixed_kernel<Q, C, 64>), grid,
                               block, args, (size_t)kWaves * 4 * TileMath<Q, C, 64, false, true>::kKSlot,
                               st);
    if (p.D == 128)
        return hipLaunchKernel(reinterpret_cast<const void*>(decode_mixed_kernel<Q, C, 128>), grid,
                               block, args, (size_t)kWaves * 4 * TileMath<Q, C, 128, false, true>::kKSlot,
                               st);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode_mixed(int qdt, int cdt, const DecodeParams& p, hipStream_t st) {
    if (!decode_mfma_supported(qdt, cdt, p.D, p.G)) return hipErrorInvalidValue;
    if (qdt == kBF16) {
        if (cdt == kFP8) return launch_mixed_d<BF16, FP8>(p, st);
        return launch_mixed_d<BF16, BF16>(p, st);
    }
    if (cdt == kFP8) return launch_mixed_d<F16, FP8>(p, st);
    return launch_mixed_d<F16, F16>(p, st);
}

bool decode_mfma_supported(int qdt, int cdt, int D, int G) {
    const bool types = (qdt == kF16 || qdt == kBF16) && (cdt == qdt || cdt == kFP8);
    return types && (D == 64 || D == 128) && G >= 1 && G <= 16;
}

hipError_t launch_decode_mfma(int qdt, int cdt, const DecodeParams& p, hipStream_t st) {
    if (!decode_mfma_supported(qdt, cdt, p.D, p.G)) return hipErrorInvalidValue;
    if (qdt == kBF16) {
        if (cdt == kFP8) return launch_d<BF16, FP8>(p, st);
        return launch_d<BF16, BF16>(p, st);
    }
    if (cdt == kFP8) return launch_d<F16, FP8>(p, st);
    return launch_d<F16, F16>(p, st);
}

}  // namespace pkv
