// prefill.hip - multi-query attention for long query runs (chunked prefill,
// "vLLM 推理引擎源码级拆解" §6.3) on 32 x 32 matrix-core tiles, with the K/V
// of a stage staged in LDS and shared by the waves of a workgroup.
//
// What is computed is that of multi_query.hip: query token i of sequence s
// sits at position L - Qn + i and attends to tokens 0 .. L - Qn + i through
// the block table; a token whose position is negative gets a zero row.
//
// Work layout.
//   - An item is one (sequence, KV head) and 256 / G consecutive query
//     tokens; each wave owns 32 of its query rows, the (token, head) pairs
//     of 32 / G tokens (GQA: the G heads of a token share the KV head, so
//     every K/V byte a wave reads feeds G rows).  A workgroup (one per CU,
//     8 waves, two per SIMD) serves two items one after the other, their
//     stages in one pipeline, so the second item's first stages load while
//     the first item's last ones are computed.
//   - The context the workgroup's last token sees is walked in stages of 64
//     keys, each wave moving 8 of them (within one block for every block
//     size).  K and V go straight from memory into one of three LDS buffers
//     (buffer loads with the LDS as destination, no registers involved):
//     stage st + 2 is requested while stage st is computed, so a stage has
//     two stages of arithmetic to arrive.  One barrier per stage.
//   - Rows are stored as in memory (no padding), their 16-byte units
//     XOR-swizzled by row against bank conflicts.  V^T operands come from
//     the gfx950 LDS transpose read.
//   - Stages all of whose keys every row of a wave sees run in a loop
//     without the causal mask, the rest in a second loop with it (one loop
//     holding both made the register allocator duplicate the accumulators).
//   - (Sequence, KV head) pairs are dealt to the XCDs round robin, an XCD
//     taking its pairs one after the other with all their groups together,
//     so the groups reading a stage share the XCD's L2.
//   - The block table entries the workgroup needs are cached in LDS.
//
// Per wave and 32-key sub-tile (v_mfma_f32_32x32x16_{bf16,f16}):
//   S^T[key][row] = K[32 x D] Q^T[D x 32]: A = K rows from LDS (lane%32 =
//     key), B = the wave's query rows held in registers (lane%32 = row).
//     The contraction over d is permuted consistently on both sides: lane
//     half g (lane / 32) supplies d in [g D/2, (g+1) D/2), 8 per
//     instruction, so each lane reads one contiguous half-row of K.
//   The result lands with lane%32 = query row and register r = key
//     8 (r/4) + 4 g + r%4, which is exactly the B layout (P^T) of
//   O^T[d][row] += V^T[d][keys] P^T[keys][row]: lane half g supplies keys
//     {4g..4g+3, 8+4g..8+4g+3} of each 16-key step, two transpose reads of
//     4 consecutive key rows each.
//   Every value of a lane's accumulators belongs to its own query row, so
//   the softmax's rescale is a per-lane multiply; the row's max and sum
//   combine the two lanes of a row (l and l ^ 32) with one lane swap.
//
// Softmax: base-2 scores (scale * log2 e folded into one FMA), lazy rescale
// (the reference max moves only when exceeded by more than 8), weights fed
// to the PV product as bf16 hi + lo (~16 significant bits) for bf16 queries
// and as f16 for f16 queries, so the only 8-bit rounding left is the stored
// output.
#include "tile_mfma.hpp"

namespace pkv {
namespace {

using namespace mfma;

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <class Q>
struct Mma32;
template <>
struct Mma32<BF16> {
    typedef __bf16 T;
    typedef bf16x8 v8;
    typedef bf16x4 v4;
    static constexpr bool kSplitP = true;
    __device__ static inline f32x16 mma(v8 a, v8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};
template <>
struct Mma32<F16> {
    typedef _Float16 T;
    typedef f16x8 v8;
    typedef f16x4 v4;
    static constexpr bool kSplitP = false;
    __device__ static inline f32x16 mma(v8 a, v8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};

constexpr int kWaves = 8;
constexpr int kRows = 32;      // query rows per wave
constexpr int kStage = 64;     // keys per LDS stage
constexpr int kSub = 32;       // keys per matrix-core sub-tile
constexpr int kBufs = 3;       // stage buffers in LDS
constexpr int kTbl = 2048;     // block table entries cached in LDS

template <int D>
struct Shape {
    static constexpr int kRow = 2 * D;                 // bytes of one head's K or V row
    static constexpr int kK = kStage * kRow;           // K of a stage
    static constexpr int kBuf = 2 * kK;                // K and V of a stage
    static constexpr int kLds = kBufs * kBuf + 2 * kTbl * 4;   // stages, two tables
    static constexpr int kChunks = kRow / 16;          // 16-byte pieces of a row
    static constexpr int kKpl = 64 / kChunks;          // keys of one wave-wide load
    static constexpr int kKpw = kStage / kWaves;       // keys each wave moves per stage
    static constexpr int kLoads = kKpw / kKpl;         // loads per wave per stage, K (and V)
    static constexpr int kQS = D / 16;                 // QK instructions (16 d each)
    static constexpr int kNT = D / 32;                 // output tiles of 32 d
    static_assert(kLoads * kKpl == kKpw && kKpw == 8, "a wave's 8 keys in whole loads");
};

// LDS serves 64 banks of 4 bytes; a 16-byte read takes 16 lanes at a
// time, an 8-byte read 32.
//
// K rows of a stage buffer (2 D bytes each): 16-byte units XORed with
// k_swizzle(row), so that the 16 rows of a score read's lanes cover all 64
// banks: row % 16 for 256-byte rows, (row / 2) % 8 for 128-byte rows (two
// rows per 64 banks).
template <int D>
__device__ inline int k_swizzle(int row) { return D == 128 ? (row & 15) : ((row >> 1) & 7); }

// V: each load's block of kKpl keys (1 KiB, CHUNKS units per key) is
// stored tile-major: unit u = 4 n + j (n the 32-column output tile, j < 4)
// of key k of the block goes to slot (k / 4) 4 CHUNKS + 16 n + 4 (k % 4) + j.
// A value read takes 8 bytes at the same columns from the 4 keys of a group
// k / 4 (the transpose read): its 32 lanes then cover 256 contiguous bytes,
// all 64 banks, and tile n is a constant 256 n bytes further.
template <int CHUNKS>
__device__ inline int v_slot(int k, int u) {
    return (k >> 2) * 4 * CHUNKS + 16 * (u >> 2) + 4 * (k & 3) + (u & 3);
}

// s_waitcnt with only a vector-memory count (expcnt and lgkmcnt at their
// maxima, so neither is waited for).
template <int N>
__device__ inline void wait_vmcnt() {
    static_assert(N >= 0 && N < 16, "vmcnt field");
    __builtin_amdgcn_s_waitcnt(0xF70 | N);
}

// The larger of x and the value of the lane 32 away (the other lane of the
// same query row), as a median with FLT_MAX: fmaxf would first quiet signalling
// NaNs of values it cannot vouch for, two more instructions, and the scores
// here are finite or -inf.
__device__ inline float row_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __builtin_amdgcn_fmed3f(__uint_as_float(r[0]), __uint_as_float(r[1]), FLT_MAX);
}

// The value fragments of one 32-key sub-tile: transpose reads (2 per
// operand; see the address sets in the kernel) from the 4 lane addresses
// a[ii][rd] (flattened) plus off, output tile n 256 n bytes further; r[ii][n][rd]
// flattened.  Each read goes through a restrict pointer, which gives it the
// alias-scope information the compiler's wait insertion needs to let it pass
// the stage loads still in flight into the other buffers (without that it
// waits for all of them before the first read).  The stage a read takes
// from is complete by the kernel's own wait and barrier either way.
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ inline u32x2 tr_read(__attribute__((address_space(3))) s16x4* __restrict__ p) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(p));
}
template <int NT>
__device__ inline void read_v_frags(u32x2 (&r)[4 * NT], const uint32_t (&a)[4], uint32_t off) {
#pragma unroll
    for (int ii = 0; ii < 2; ii++)
#pragma unroll
        for (int n = 0; n < NT; n++)
#pragma unroll
            for (int rd = 0; rd < 2; rd++)
                r[ii * 2 * NT + 2 * n + rd] = tr_read(
                    (__attribute__((address_space(3))) s16x4*)(size_t)(a[2 * ii + rd] + off + 256 * n));
}

template <class Q, int D>
__global__ __launch_bounds__(64 * kWaves, 2) void prefill_kernel(DecodeParams p) {
    typedef Shape<D> SH;
    typedef Mma32<Q> M;
    typedef typename M::T T;
    typedef typename M::v8 v8;
    extern __shared__ __attribute__((aligned(16))) char lds[];
    int* tbl_lds = (int*)(lds + kBufs * SH::kBuf);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int c = lane & 31;               // this lane's query row within the wave
    const int g = lane >> 5;               // lane half
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    // workgroup -> two items (sequence, KV head, group of query tokens).
    // Workgroups are dealt to the XCDs in turn (blockIdx % 8), and the
    // (sequence, KV head) pairs round robin to the XCDs (pair % 8), so each
    // XCD gets a share of every sequence's work.  Within an XCD of n items,
    // workgroup j (the j-th dispatched there) takes the j-th longest item
    // (by the keys it reads) and then the (n - 1 - j)-th: the longest with
    // the shortest, which is where the longest-first rule for jobs on
    // identical machines puts the second item of each CU when n is twice
    // the CUs.  Items of one pair differ by a group's tokens, so a pair's
    // groups run close together and share the stages in the XCD's L2.
    // Every workgroup ranks the items itself (at most 512 per XCD, one per
    // thread); with more, pair by pair, the longest group first.
    const int G = p.G;
    const int tpw = kRows / G;             // query tokens per wave
    const int tpg = kWaves * tpw;          // per workgroup
    const int pairs = p.S * p.Hkv;
    const int xcd = (int)(blockIdx.x % 8);
    const int j = (int)(blockIdx.x / 8);
    const int n_items = (pairs > xcd ? (pairs - xcd + 7) / 8 : 0) * p.max_groups;
    if (j >= (n_items + 1) / 2) return;    // whole workgroup
    // the workgroup's two items: ranks j and n_items - 1 - j
    int itemA = j, itemB = n_items - 1 - j > j ? n_items - 1 - j : -1;
    if (n_items <= 64 * kWaves) {
        int* key = tbl_lds;                // the tables' space, free until filled
        int w = -1;
        if (tid < n_items) {
            const int ps = ((tid / p.max_groups) * 8 + xcd) / p.Hkv;
            const int qn = p.q_start[ps + 1] - p.q_start[ps];
            const int base = (p.max_groups - 1 - tid % p.max_groups) * tpg;
            if (base < qn) {
                const int Ls = min(p.lens[ps], p.len_cap);
                w = max(0, Ls - qn + min(base + tpg, qn));
            }
            key[tid] = w;
        }
        if (tid == 0) key[kTbl - 2] = -1;
        __syncthreads();
        if (tid < n_items) {
            int rank = 0;
            for (int k = 0; k < n_items; k++) {
                const int wk = key[k];
                rank += (wk > w) | ((wk == w) & (k < tid));
            }
            if (rank == j) key[kTbl - 1] = tid;
            if (rank == n_items - 1 - j && rank != j) key[kTbl - 2] = tid;
        }
        __syncthreads();
        itemA = __builtin_amdgcn_readfirstlane(key[kTbl - 1]);
        itemB = __builtin_amdgcn_readfirstlane(key[kTbl - 2]);
        __syncthreads();                   // before the tables are filled
    }
    // An item: (sequence, KV head, group of query tokens), wave-uniform.
    // nstage = 0 for an item without keys; valid = 0 for one without rows.
    struct Item {
        int s, h, q0, Qn, L, wg_base, wg_end, nblk, nstage, tb0, valid;
    };
    const int bs_shift = p.bs == 8 ? 3 : (p.bs == 16 ? 4 : 5);
    auto make_item = [&](int item) {
        Item it;
        it.s = it.h = it.q0 = it.Qn = it.L = it.wg_base = 0;
        it.wg_end = it.nblk = it.nstage = it.tb0 = it.valid = 0;
        if (item < 0) return it;
        const int pair = (item / p.max_groups) * 8 + xcd;
        const int grp = p.max_groups - 1 - item % p.max_groups;
        if (pair >= pairs) return it;
        it.h = pair % p.Hkv;
        it.s = pair / p.Hkv;
        it.q0 = __builtin_amdgcn_readfirstlane(p.q_start[it.s]);
        it.Qn = __builtin_amdgcn_readfirstlane(p.q_start[it.s + 1]) - it.q0;
        it.wg_base = grp * tpg;
        if (it.wg_base >= it.Qn) return it;
        int L = __builtin_amdgcn_readfirstlane(p.lens[it.s]);
        it.L = L < p.len_cap ? L : p.len_cap;
        // keys the workgroup's last query token sees (0: none)
        it.wg_end = max(0, it.L - it.Qn + min(it.wg_base + tpg, it.Qn));
        it.nblk = it.wg_end > 0 ? ((it.wg_end - 1) >> bs_shift) + 1 : 0;
        it.nstage = (it.wg_end + kStage - 1) / kStage;
        it.valid = 1;
        return it;
    };
    Item A = make_item(itemA), B = make_item(itemB);

    // ---- this lane's query row (of the current item) ----
    const int hh = c % G;
    int tok = 0, pos = 0, lim = INT_MAX, wlast = -1, wvis = INT_MAX;
    bool has_row = false, sees = false;
    // Scores enter the exponent as fma(s, |scale'|, -m); a negative scale is
    // carried by the query's sign (exact).
    const float sl2 = p.scale_log2;
    const float sla = fabsf(sl2);
    v8 qf[SH::kQS];
    auto setup_rows = [&](const Item& it) {
        tok = it.wg_base + wave * tpw + c / G;          // query token within the sequence
        has_row = it.valid && tok < it.Qn;
        pos = it.L - it.Qn + tok;                       // its position in the sequence
        sees = has_row && pos >= 0;
        // last key this row sees; rows that see nothing read everything (zero
        // queries, never written), which keeps every row's max finite
        lim = sees ? pos : INT_MAX;
        const T* qrow = (const T*)p.q + ((size_t)(it.q0 + (sees ? tok : 0)) * p.Hq +
                                         (size_t)it.h * G + hh) * D;
        const uint32_t flip = sl2 < 0.0f ? 0x80008000u : 0u;
#pragma unroll
        for (int i = 0; i < SH::kQS; i++) {
            u32x4 x = sees ? *(const u32x4*)(qrow + (D / 2) * g + 8 * i) : u32x4{};
            x ^= flip;
            qf[i] = __builtin_bit_cast(v8, x);
        }
        // wave-uniform bounds over the rows that see keys: the last key any
        // of them sees, and the last key all of them see
        int wl = sees ? pos : -1;
        int wv = sees ? pos : INT_MAX;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            wl = max(wl, __shfl_xor(wl, o, 64));
            wv = min(wv, __shfl_xor(wv, o, 64));
        }
        wlast = __builtin_amdgcn_readfirstlane(wl);
        wvis = __builtin_amdgcn_readfirstlane(wv);
    };

    // ---- block table entries in LDS ----
    // Entries [tb0, tb0 + kTbl) of each item's table, item A's in the first
    // kTbl words, B's in the next; a stage whose blocks pass the end has the
    // next kTbl loaded first (all waves, at a stage boundary: rare, a
    // 2048-block span).
    int* tblA = tbl_lds;
    int* tblB = tbl_lds + kTbl;
    auto fill_table = [&](int* dst, const Item& it, int b0) {
        const int32_t* table = p.tables + (size_t)it.s * p.max_blocks;
        for (int i = tid; i < kTbl; i += 64 * kWaves)
            dst[i] = b0 + i < it.nblk ? table[b0 + i] : 0;
    };

    // ---- stage loads ----
    // Wave w moves keys 8 w .. 8 w + 7 of a stage (one block: block sizes
    // are multiples of 8), so its table entry is wave-uniform and every
    // load has a scalar buffer descriptor.  Load r covers keys 8 w + kKpl r
    // .. + kKpl - 1, lane i writing 16 bytes at i * 16 from the load's
    // first byte.  K: row i / kChunks, unit (i % kChunks) ^ k_swizzle(row)
    // of the key's row.  V: lane i fills slot i of the tile-major block.
    // Keys at or past wg_end take an out-of-range offset and write zeros.
    const uint32_t pool_row = (uint32_t)p.Hkv * SH::kRow;       // bytes between slots
    const uint32_t blk_bytes = (uint32_t)p.bs * pool_row;
    const int lj = lane / SH::kChunks;
    const int ch = lane % SH::kChunks;
    // the V slot this lane fills (v_slot inverted): key vk of the block, unit vu
    const int vrem = lane % (4 * SH::kChunks);
    const int vk = 4 * (lane / (4 * SH::kChunks)) + ((vrem >> 2) & 3);
    const int vu = 4 * (vrem >> 4) + (vrem & 3);
    auto load_stage = [&](const Item& it, const int* tbl, int st, int buf) {
        const uint32_t head_off = (uint32_t)it.h * SH::kRow;
        const int wg_end = it.wg_end;
        const int t0 = st * kStage + SH::kKpw * wave;
        const int e = tbl[min(t0 >> bs_shift, it.nblk - 1) - it.tb0];
        const uint32_t b0 = (uint32_t)__builtin_amdgcn_readfirstlane(e);
        const uint32_t b = b0 < (uint32_t)p.NB ? b0 : (uint32_t)p.NB - 1u;
        const rsrc_t rk = make_rsrc((const char*)p.k + (size_t)b * blk_bytes, blk_bytes);
        const rsrc_t rv = make_rsrc((const char*)p.v + (size_t)b * blk_bytes, blk_bytes);
        char* kdst = lds + buf * SH::kBuf + SH::kKpw * wave * SH::kRow;
        char* vdst = kdst + SH::kK;
#pragma unroll
        for (int r = 0; r < SH::kLoads; r++) {
            const int row0 = SH::kKpw * wave + r * SH::kKpl;     // within the stage
            const int dst = r * SH::kKpl * SH::kRow;
            const int tk = st * kStage + row0 + lj;
            const uint32_t uk = (uint32_t)(ch ^ k_swizzle<D>(row0 + lj));
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rk, (__attribute__((address_space(3))) void*)(kdst + dst), 16,
                tk < wg_end ? (uint32_t)(tk & (p.bs - 1)) * pool_row + head_off + 16u * uk : kOOB,
                0, 0, 0);
            const int tv = st * kStage + row0 + vk;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rv, (__attribute__((address_space(3))) void*)(vdst + dst), 16,
                tv < wg_end ? (uint32_t)(tv & (p.bs - 1)) * pool_row + head_off + 16u * vu : kOOB,
                0, 0, 0);
        }
    };

    // ---- running state of this lane's row ----
    f32x16 o[SH::kNT];
#pragma unroll
    for (int n = 0; n < SH::kNT; n++) o[n] = f32x16{};
    float m = -INFINITY, l = 0.0f;   // reference max (scaled, base 2) and sum

    // Lane-constant LDS addresses of the operand reads, relative to a stage
    // buffer.  K: row c of a sub-tile, unit (D / 16) g + i of the score
    // step i, swizzled.
    uint32_t ka[SH::kQS];
#pragma unroll
    for (int i = 0; i < SH::kQS; i++)
        ka[i] = (uint32_t)(c * SH::kRow) + (uint32_t)((((D / 16) * g + i) ^ k_swizzle<D>(c)) << 4);
    // V^T fragments by transpose reads.  Two reads per operand (rd 0: keys
    // 4g..4g+3, rd 1: keys 8+4g..8+4g+3 of the 16-key step ii); in lane
    // group G16 = lane / 16 (half g = G16 / 2, 16 columns from 32 n + 16
    // (G16 % 2)), lane s = 4 mr + tc addresses key mr of the four and
    // columns 4 tc .. 4 tc + 3: unit 2 (G16 % 2) + tc / 2 of tile n, half
    // tc % 2 of it.  The four keys start a V block's group of four.
    uint32_t va[2][2];
    {
        const int G16 = lane >> 4, sl = lane & 15, mr = sl >> 2, tc = sl & 3;
#pragma unroll
        for (int ii = 0; ii < 2; ii++)
#pragma unroll
            for (int rd = 0; rd < 2; rd++) {
                const int key = 16 * ii + 8 * rd + 4 * g + mr;
                const int blk = key / SH::kKpl;
                const int slot = v_slot<SH::kChunks>(key % SH::kKpl, 2 * (G16 & 1) + (tc >> 1));
                va[ii][rd] = (uint32_t)(SH::kK + blk * SH::kKpl * SH::kRow + 16 * slot + 8 * (tc & 1));
            }
    }

    // One 32-key sub-tile u of the stage in LDS buffer `base`: scores, the
    // softmax update, the value products.
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    // the sum of the 8 pairs of 16-bit weights in w (one per dot product)
    auto sum_words = [](const uint32_t (&w)[2][4]) {
        float t = 0.0f;
#pragma unroll
        for (int ii = 0; ii < 2; ii++)
#pragma unroll
            for (int q = 0; q < 4; q++) {
                if constexpr (M::kSplitP)
                    t = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[ii][q]),
                                                        bf16x2{(__bf16)1.0f, (__bf16)1.0f}, t, false);
                else
                    t = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w[ii][q]),
                                               f16x2{(_Float16)1.0f, (_Float16)1.0f}, t, false);
            }
        return t;
    };
    auto sub_tile = [&](const char* base, int u, int kb, auto mask) {
        constexpr bool MASK = decltype(mask)::value;
        // all K fragments requested before the first product
        v8 kf[SH::kQS];
#pragma unroll
        for (int i = 0; i < SH::kQS; i++)
            kf[i] = *(const v8*)(base + ka[i] + u * kSub * SH::kRow);
        // keep all the reads ahead of the products (otherwise the scheduler
        // reuses one register tuple and waits for each read in turn)
        __builtin_amdgcn_sched_barrier(0);
        f32x16 sc = f32x16{};
#pragma unroll
        for (int i = 0; i < SH::kQS; i++) sc = M::mma(kf[i], qf[i], sc);
        // the value fragments, read while the score products run
        v8 vf[2][SH::kNT];
        {
            const uint32_t sb = (uint32_t)(size_t)(__attribute__((address_space(3))) const char*)base;
            uint32_t a[4];
#pragma unroll
            for (int i = 0; i < 4; i++) a[i] = sb + (&va[0][0])[i];
            u32x2 r[4 * SH::kNT];
            read_v_frags<SH::kNT>(r, a, (uint32_t)(u * kSub * SH::kRow));
#pragma unroll
            for (int ii = 0; ii < 2; ii++)
#pragma unroll
                for (int n = 0; n < SH::kNT; n++) {
                    const u32x2 lo = r[ii * 2 * SH::kNT + 2 * n], hi = r[ii * 2 * SH::kNT + 2 * n + 1];
                    vf[ii][n] = __builtin_bit_cast(v8, u32x4{lo[0], lo[1], hi[0], hi[1]});
                }
        }

        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; r++) {
            const int key = kb + 8 * (r >> 2) + 4 * g + (r & 3);
            mx = fmaxf(mx, (!MASK || key <= lim) ? sc[r] : -INFINITY);
        }
        mx = row_max(mx);
        // a row that sees no key of the sub-tile keeps -inf (not -inf * sla)
        const float mxs = MASK && mx == -INFINITY ? -INFINITY : mx * sla;
        const float m_new = mxs > m + mfma::kTau ? mxs : m;
        if (__any(m_new != m)) {
            const float alpha = m_new == m ? 1.0f : __builtin_amdgcn_exp2f(m - m_new);
            l *= alpha;
#pragma unroll
            for (int n = 0; n < SH::kNT; n++) o[n] *= alpha;
            m = m_new;
        }
        const float nm = -m;
        float pz[16];
#pragma unroll
        for (int r = 0; r < 16; r++) {
            const float e = __builtin_amdgcn_exp2f(fmaf(sc[r], sla, nm));
            const int key = kb + 8 * (r >> 2) + 4 * g + (r & 3);
            pz[r] = (!MASK || key <= lim) ? e : 0.0f;
        }
        // element e of the operand of step ii is score register 8 ii + e
        // (keys 4g.. and 8 + 4g.. of the step, the order of the value reads)
        uint32_t hw[2][4];
#pragma unroll
        for (int ii = 0; ii < 2; ii++)
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const f32x2 x = {pz[8 * ii + 2 * q], pz[8 * ii + 2 * q + 1]};
                if constexpr (M::kSplitP)
                    hw[ii][q] = __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
                else
                    hw[ii][q] = __builtin_bit_cast(uint32_t, __builtin_convertvector(x, f16x2));
            }
        // The running sum takes the 16-bit weights themselves, the numbers
        // the value products see, two per dot product with (1, 1): the
        // output is then a weighted mean with exactly its own weights.
        l += sum_words(hw);
#pragma unroll
        for (int ii = 0; ii < 2; ii++) {
            const v8 hi = __builtin_bit_cast(v8, u32x4{hw[ii][0], hw[ii][1], hw[ii][2], hw[ii][3]});
#pragma unroll
            for (int n = 0; n < SH::kNT; n++) o[n] = M::mma(vf[ii][n], hi, o[n]);
        }
        if constexpr (M::kSplitP) {
            // bf16 keeps 8 significant bits of a weight.  A lane whose
            // largest weight here (at most that of its row's best key)
            // exceeds 1/8 of its running sum also feeds the remainder
            // p - bf16(p) (another 8 bits); below that share every weight
            // ends at most 1/8 of the row's total, and the rounding of many
            // such small weights stays far inside the tolerance.  The
            // decision is the lane's own, so a row's arithmetic does not
            // depend on the other rows of the wave.
            const bool fine = __builtin_amdgcn_exp2f(mxs - m) > 0.125f * l;
            if (__any(fine)) {
                uint32_t lws[2][4];
#pragma unroll
                for (int ii = 0; ii < 2; ii++) {
                    uint32_t lw[4];
#pragma unroll
                    for (int q = 0; q < 4; q++) {
                        const f32x2 x = {pz[8 * ii + 2 * q], pz[8 * ii + 2 * q + 1]};
                        const f32x2 hv = {__builtin_bit_cast(float, hw[ii][q] << 16),
                                          __builtin_bit_cast(float, hw[ii][q] & 0xFFFF0000u)};
                        const uint32_t r =
                            __builtin_bit_cast(uint32_t, __builtin_convertvector(x - hv, bf16x2));
                        lw[q] = fine ? r : 0u;
                    }
                    const v8 lo = __builtin_bit_cast(v8, u32x4{lw[0], lw[1], lw[2], lw[3]});
#pragma unroll
                    for (int n = 0; n < SH::kNT; n++) o[n] = M::mma(vf[ii][n], lo, o[n]);
                    lws[ii][0] = lw[0], lws[ii][1] = lw[1], lws[ii][2] = lw[2], lws[ii][3] = lw[3];
                }
                l += sum_words(lws);        // zero words where the lane is not fine
            }
        }
    };

    // ---- the stage pipeline ----
    // The stages of item A and then those of item B form one sequence
    // (global stage gg).  At the top of stage gg the loads of stage gg + 2
    // are issued into buffer (gg + 2) % 3, last read during stage gg - 1
    // (every wave has passed the barrier that ended it); so B's first two
    // stages arrive while A's last two are computed.  At the bottom, the
    // wave waits for its loads of stage gg + 1 (all but the kLoads K and
    // kLoads V loads of stage gg + 2, issued after them, in order) and meets
    // the others: past that barrier every wave's rows of stage gg + 1 are in
    // LDS.
    const int NA = A.nstage, NT = A.nstage + B.nstage;
    // loads of stage st of item X, after the table span holding its blocks
    // (workgroup-uniform)
    auto issue_item = [&](Item& X, int* tbl, int st, int buf) {
        const int last = min(((st + 1) * kStage - 1) >> bs_shift, X.nblk - 1);
        if (last >= X.tb0 + kTbl) {
            wait_vmcnt<0>();
            __syncthreads();
            X.tb0 = (st * kStage) >> bs_shift;
            fill_table(tbl, X, X.tb0);
            __syncthreads();
        }
        load_stage(X, tbl, st, buf);
    };
    auto issue = [&](int gg) {
        if (gg < NA) issue_item(A, tblA, gg, gg % kBufs);
        else if (gg < NT) issue_item(B, tblB, gg - NA, gg % kBufs);
    };
    setup_rows(A);
    fill_table(tblA, A, 0);
    if (B.valid) fill_table(tblB, B, 0);
    __syncthreads();
    issue(0);
    issue(1);
    wait_vmcnt<0>();                       // stages 0 and 1 in LDS
    __builtin_amdgcn_s_barrier();
    // Stages [st0, st1) of the item whose first stage is goff, every
    // sub-tile with the causal limits (MASK) or, for stages all of whose
    // keys every row of the wave sees, without.  Every stage passes one
    // barrier, so waves that split the stages differently still meet at
    // each one.
    auto run_stages = [&](int goff, int st0, int st1, auto mask) {
        for (int st = st0; st < st1; st++) {
            const int gg = goff + st;
            issue(gg + 2);
            const char* base = lds + (gg % kBufs) * SH::kBuf;
#pragma unroll
            for (int u = 0; u < kStage / kSub; u++) {
                const int kb = st * kStage + u * kSub;
                if (kb <= wlast) sub_tile(base, u, kb, mask);            // wave-uniform
            }
            // stage gg + 1 in LDS: at most the 2 kLoads loads of stage
            // gg + 2 may still be in flight
            if (gg + 2 < NT) wait_vmcnt<2 * SH::kLoads>();
            else wait_vmcnt<0>();
            __builtin_amdgcn_s_barrier();
        }
    };
    // normalise and store this lane's row of item `it`
    auto epilogue = [&](const Item& it) {
        if (has_row) {
            const float l_tot = swap_sum32(l);
            const float inv = sees && l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
            T* orow = (T*)p.out + ((size_t)(it.q0 + tok) * p.Hq + (size_t)it.h * G + hh) * D;
            typedef T t4 __attribute__((ext_vector_type(4)));
#pragma unroll
            for (int n = 0; n < SH::kNT; n++)
#pragma unroll
                for (int rq = 0; rq < 4; rq++) {
                    t4 v;
#pragma unroll
                    for (int e = 0; e < 4; e++) v[e] = (T)(o[n][4 * rq + e] * inv);
                    *(t4*)(orow + 32 * n + 8 * rq + 4 * g) = v;
                }
        }
    };
    // stage st of an item is seen whole by every row of the wave when
    // st * kStage + kStage - 1 <= wvis (wvis is INT_MAX for a wave without
    // rows: it computes nothing and only passes the barriers)
    {
        const int nfull = (int)min64(NA, ((int64_t)wvis + 1) / kStage);
        run_stages(0, 0, nfull, std::false_type{});
        run_stages(0, nfull, NA, std::true_type{});
        epilogue(A);
    }
    if (B.valid) {
        setup_rows(B);
#pragma unroll
        for (int n = 0; n < SH::kNT; n++) o[n] = f32x16{};
        m = -INFINITY;
        l = 0.0f;
        const int nfull = (int)min64(B.nstage, ((int64_t)wvis + 1) / kStage);
        run_stages(NA, 0, nfull, std::false_type{});
        run_stages(NA, nfull, B.nstage, std::true_type{});
        epilogue(B);
    }
}

template <class Q, int D>
hipError_t launch_dd(const DecodeParams& p, hipStream_t st) {
    typedef Shape<D> SH;
    const long pairs = (long)p.S * p.Hkv;
    const long per_xcd = (pairs + 7) / 8 * p.max_groups;    // items of XCD 0 (the most)
    const long wgs = 8 * ((per_xcd + 1) / 2);               // two items per workgroup
    void* args[] = {const_cast<DecodeParams*>(&p)};
    return hipLaunchKernel(reinterpret_cast<const void*>(prefill_kernel<Q, D>),
                           dim3((unsigned)wgs), dim3(64 * kWaves), args, SH::kLds, st);
}

}  // namespace

// Query tokens one prefill workgroup serves: 32 query rows per wave.
int prefill_tokens_per_group(int G) { return kWaves * (kRows / G); }

bool prefill_supported(int qdt, int cdt, int D, int G) {
    return (qdt == kF16 || qdt == kBF16) && cdt == qdt && (D == 64 || D == 128) && G >= 1 &&
           G <= 16 && (G & (G - 1)) == 0;
}

hipError_t launch_prefill(int qdt, int cdt, const DecodeParams& p, hipStream_t st) {
    if (!prefill_supported(qdt, cdt, p.D, p.G)) return hipErrorInvalidValue;
    if (qdt == kBF16) {
        if (p.D == 64) return launch_dd<BF16, 64>(p, st);
        return launch_dd<BF16, 128>(p, st);
    }
    if (p.D == 64) return launch_dd<F16, 64>(p, st);
    return launch_dd<F16, 128>(p, st);
}

}  // namespace pkv
