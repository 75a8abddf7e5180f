// prefill.hip - multi-query attention for long query runs (chunked prefill,
// "vLLM 推理引擎源码级拆解" §6.3) with the K/V tiles staged in LDS and
// shared by the waves of a workgroup.
//
// What is computed is that of multi_query.hip: query token i of sequence s
// sits at position L - Qn + i and attends to tokens 0 .. L - Qn + i through
// the block table.  The work is laid out for reuse of K/V:
//   - a workgroup serves one (sequence, KV head) and kTok consecutive query
//     tokens; each of its kWaves waves carries NB column blocks of the
//     matrix-core tile (16 / G tokens x G heads each), as the wide kernel of
//     multi_query.hip does;
//   - the context the workgroup's last token sees is walked in stages of
//     kStageTok tokens: all threads load a stage's K and V rows (through
//     the block table, with buffer loads; rows past the context read as
//     zeros) into one of two LDS buffers, one barrier per stage, and every
//     wave reads its 16-token
//     tiles from LDS in the lane layout of tile_mfma.hpp and runs the same
//     causal tile step;
//   - the next stage's rows are loaded into registers while the current one
//     is computed, and written to the other buffer after it.
// So a 512-token chunk reads its context from memory once per kTok query
// tokens instead of once per wave, and the waves hold no ring of tiles in
// flight: at two column blocks per wave two waves fit on a SIMD.  The tile
// step is bound by vector instructions, so a wave widens and permutes a
// tile's value rows once for both its column blocks, and skips the causal
// mask on tiles every one of its columns sees whole (all but the last few
// of a long context).
// LDS rows are padded by 16 bytes so that the 16 rows a tile's K slices come
// from fall in distinct banks.
#include "tile_mfma.hpp"

namespace pkv {
namespace {

using namespace mfma;

constexpr int kWaves = 4;
constexpr int kStageTok = 64;              // tokens per LDS stage (4 tiles)

template <class Q, class C, int D, int NB>
struct PrefillShape {
    static constexpr int EB = C::kBytes;
    static constexpr int kRow = D * EB;                    // bytes of one head's row
    static constexpr int kStride = kRow + 16;              // padded LDS row
    static constexpr int kHalf = kStageTok * kStride;      // K (or V) rows of a stage
    static constexpr int kBuf = 2 * kHalf;                 // K and V of a stage
    static constexpr int kLds = 2 * kBuf;                  // double buffer
    static constexpr int kChunks = kRow / 16;              // 16-byte pieces per row
    // 16-byte loads per thread per stage (K and V rows)
    static constexpr int kLoads = 2 * kStageTok * kChunks / (64 * kWaves);
    static_assert(kLoads * 64 * kWaves == 2 * kStageTok * kChunks, "stage split");
};

template <class Q, class C, int D, int NB>
__global__ __launch_bounds__(64 * kWaves, 2) void prefill_kernel(DecodeParams p) {
    typedef TileMath<Q, C, D, false> TM;
    typedef PrefillShape<Q, C, D, NB> SH;
    typedef typename TM::T T;
    typedef typename TM::v8 v8;
    typedef typename TM::vraw vraw;
    extern __shared__ __attribute__((aligned(16))) char lds[];
    const TM tm;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    // workgroup -> (sequence, KV head, group of query tokens)
    const int G = p.G;
    const int QPG = 16 / G;
    const int kTok = kWaves * NB * QPG;                    // query tokens per workgroup
    const int grp = blockIdx.x % p.max_groups;
    const int h = (blockIdx.x / p.max_groups) % p.Hkv;
    const int s = blockIdx.x / p.max_groups / p.Hkv;
    if (s >= p.S) return;                                  // whole workgroup
    const int q0 = __builtin_amdgcn_readfirstlane(p.q_start[s]);
    const int Qn = __builtin_amdgcn_readfirstlane(p.q_start[s + 1]) - q0;
    const int wg_base = grp * kTok;
    if (wg_base >= Qn) return;                             // whole workgroup
    int L = __builtin_amdgcn_readfirstlane(p.lens[s]);
    L = L < p.len_cap ? L : p.len_cap;
    // tokens the workgroup's last query token sees
    const int wg_end = L - Qn + min(kTok, Qn - wg_base) + wg_base;

    // this wave's query tokens
    const int qbase = wg_base + wave * NB * QPG;
    const int nq = max(0, min(NB * QPG, Qn - qbase));
    const int t_end = nq > 0 ? L - Qn + qbase + nq : 0;    // tokens its last one sees
    auto out_row = [&](int b, int c) {
        return (T*)p.out +
               ((size_t)(q0 + qbase + b * QPG + c / G) * p.Hq + (size_t)h * G + c % G) * D;
    };

    v8 qb[NB][TM::KS];
    int pc[NB], ncols[NB];
#pragma unroll
    for (int b = 0; b < NB; b++) {
        const int tb = qbase + b * QPG;
        const int nqb = max(0, min(QPG, Qn - tb));
        ncols[b] = nqb * G;
        const T* qrow = (const T*)p.q +
                        ((size_t)(q0 + tb + tm.j16 / G) * p.Hq + (size_t)h * G + tm.j16 % G) * D;
#pragma unroll
        for (int kk = 0; kk < TM::KS; kk++) {
            const int d0 = 32 * kk + 8 * tm.g4;
            qb[b][kk] = tm.j16 < ncols[b] ? *(const v8*)(qrow + d0) : v8{};
        }
        pc[b] = tm.j16 < ncols[b] ? L - Qn + tb + tm.j16 / G : -1;
    }
    typename TM::Acc acc[NB];
#pragma unroll
    for (int b = 0; b < NB; b++) tm.reset(acc[b]);
    // The last token every live column of this wave sees: tiles up to it
    // need no causal mask (columns past the wave's tokens are never written).
    int vis = INT_MAX;
#pragma unroll
    for (int b = 0; b < NB; b++) vis = min(vis, tm.j16 < ncols[b] ? pc[b] : INT_MAX);
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) vis = min(vis, __shfl_xor(vis, o, 64));
    vis = __builtin_amdgcn_readfirstlane(vis);

    // ---- stage loads: thread tid moves kLoads 16-byte pieces per stage ----
    const int32_t* table = p.tables + (size_t)s * p.max_blocks;
    const int bs_shift = p.bs == 8 ? 3 : (p.bs == 16 ? 4 : 5);
    const size_t pool_row = (size_t)p.Hkv * SH::kRow;      // bytes between slots
    const size_t head_off = (size_t)h * SH::kRow;
    u32x4 stage[SH::kLoads];
    // Piece j of thread tid is K (or V) row t, 16-byte chunk tid % kChunks.
    // The 64 lanes of a wave cover 64 / kChunks consecutive, aligned rows
    // (4 at D = 128, 8 at D = 64), so they lie in one block for every block
    // size: one wave-uniform table entry (a scalar load) and one buffer
    // descriptor per piece.  Rows at or past wg_end take an offset past the
    // descriptor and read zeros, with no branch around the load (a branch
    // would make the loop wait for every load in flight).
    static_assert(64 % SH::kChunks == 0 && 64 / SH::kChunks <= 8, "a wave's rows in one block");
    const int lane_row = (tid & 63) / SH::kChunks;
    const uint32_t lane_chunk = (uint32_t)((tid & 63) % SH::kChunks) * 16u;
    const uint32_t blk_bytes = (uint32_t)p.bs * (uint32_t)pool_row;
    auto load_stage = [&](int t0) {
        // the wave's first row of piece j
        auto row0 = [&](int j) {
            return t0 + ((j * 64 * kWaves + wave * 64) % (kStageTok * SH::kChunks)) / SH::kChunks;
        };
        uint32_t blk[SH::kLoads];
#pragma unroll
        for (int j = 0; j < SH::kLoads; j++)   // all table entries first, one wait
            blk[j] = (uint32_t)table[min(row0(j), wg_end - 1) >> bs_shift];
#pragma unroll
        for (int j = 0; j < SH::kLoads; j++) {
            const int kv = (j * 64 * kWaves + wave * 64) / (kStageTok * SH::kChunks);   // 0: K, 1: V
            const int tw = row0(j);
            const uint32_t b = blk[j] < (uint32_t)p.NB ? blk[j] : (uint32_t)p.NB - 1u;
            const rsrc_t r = make_rsrc((const char*)(kv ? p.v : p.k) + (size_t)b * blk_bytes,
                                       blk_bytes);
            const int t = tw + lane_row;
            const uint32_t off = t < wg_end ? (uint32_t)(t & (p.bs - 1)) * (uint32_t)pool_row +
                                                  (uint32_t)head_off + lane_chunk
                                            : kOOB;
            stage[j] = Buf<16>::load(r, off);
        }
    };
    auto store_stage = [&](int buf) {
        char* dst = lds + buf * SH::kBuf;
#pragma unroll
        for (int j = 0; j < SH::kLoads; j++) {
            const int idx = j * 64 * kWaves + tid;
            const int kv = idx / (kStageTok * SH::kChunks);
            const int rem = idx % (kStageTok * SH::kChunks);
            *(u32x4*)(dst + kv * SH::kHalf + (rem / SH::kChunks) * SH::kStride +
                      (rem % SH::kChunks) * 16) = stage[j];
        }
    };
    // tile j16-row layout of tile_mfma.hpp, read from a stage in LDS
    auto read_tile = [&](int buf, int tile, typename TM::Tile& tl) {
        const char* kb = lds + buf * SH::kBuf + tile * 16 * SH::kStride;
        const char* vb = kb + SH::kHalf;
#pragma unroll
        for (int i = 0; i < TM::KL; i++)
            tl.k[i] = *(const u32x4*)(kb + tm.j16 * SH::kStride + tm.kcol[i]);
#pragma unroll
        for (int r = 0; r < 4; r++)
            tl.v[r] = *(const vraw*)(vb + (4 * tm.g4 + r) * SH::kStride + tm.vcol);
    };

    const int nstage = (wg_end + kStageTok - 1) / kStageTok;   // >= 1 when wg_end > 0
    if (nstage > 0) {
        load_stage(0);
        store_stage(0);
    }
    __syncthreads();
    // Stages [st0, st1), every tile with the causal limits (MASK) or, for
    // stages all of whose tokens every column of this wave sees, without.
    // Each call passes one barrier per stage, so waves that split the
    // stages differently still meet at every barrier.
    auto run_stages = [&](int st0, int st1, auto mask) {
        constexpr bool MASK = decltype(mask)::value;
        for (int st = st0; st < st1; st++) {
            const int buf = st & 1;
            const int t0 = st * kStageTok;
            const bool more = st + 1 < nstage;
            if (more) load_stage(t0 + kStageTok);          // in flight during the tiles
#pragma unroll
            for (int tile = 0; tile < kStageTok / 16; tile++) {
                const int tt = t0 + 16 * tile;
                if (tt < t_end) {                          // wave-uniform
                    typename TM::Tile tl;
                    read_tile(buf, tile, tl);
#pragma unroll
                    for (int b = NB - 1; b >= 0; b--)
                        tm.template consume<true, MASK>(acc[b], qb[b], p.scale_log2,
                                                        t_end - 1 - tt, tl, pc[b] - tt);
                }
            }
            if (more) store_stage(buf ^ 1);                // read by no wave since the
            __syncthreads();                               // last barrier
        }
    };
    // stage st is seen whole by every live column when st * kStageTok +
    // kStageTok - 1 <= vis.  A wave with no live column (nq == 0, the tail
    // of a ragged chunk) consumes no tile and only passes the barriers; its
    // vis is still INT_MAX, so the count is taken in 64 bits.
    const int nfull =
        vis >= kStageTok - 1 ? (int)min64(nstage, ((int64_t)vis + 1) / kStageTok) : 0;
    run_stages(0, nfull, std::false_type{});
    run_stages(nfull, nstage, std::true_type{});

#pragma unroll
    for (int b = 0; b < NB; b++)
        tm.finish_each(
            acc[b], ncols[b], [&](int) { return true; }, p.v_scale,
            [&](int c) { return out_row(b, c); }, [&](int) { return (float*)nullptr; },
            [&](int) { return (float*)nullptr; }, [&](int) { return (float*)nullptr; });
}

template <class Q, class C, int D>
hipError_t launch_dd(const DecodeParams& p, hipStream_t st) {
    constexpr int NB = 2;
    typedef PrefillShape<Q, C, D, NB> SH;
    const long wgs = (long)p.S * p.Hkv * p.max_groups;
    void* args[] = {const_cast<DecodeParams*>(&p)};
    return hipLaunchKernel(reinterpret_cast<const void*>(prefill_kernel<Q, C, D, NB>),
                           dim3((unsigned)wgs), dim3(64 * kWaves), args, SH::kLds, st);
}

}  // namespace

// Query tokens one prefill workgroup serves.
int prefill_tokens_per_group(int G) { return kWaves * 2 * (16 / G); }

bool prefill_supported(int qdt, int cdt, int D, int G) {
    return (qdt == kF16 || qdt == kBF16) && cdt == qdt && (D == 64 || D == 128) && G >= 1 &&
           G <= 16;
}

hipError_t launch_prefill(int qdt, int cdt, const DecodeParams& p, hipStream_t st) {
    if (!prefill_supported(qdt, cdt, p.D, p.G)) return hipErrorInvalidValue;
    if (qdt == kBF16) {
        if (p.D == 64) return launch_dd<BF16, BF16, 64>(p, st);
        return launch_dd<BF16, BF16, 128>(p, st);
    }
    if (p.D == 64) return launch_dd<F16, F16, 64>(p, st);
    return launch_dd<F16, F16, 128>(p, st);
}

}  // namespace pkv
