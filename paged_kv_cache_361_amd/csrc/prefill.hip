// prefill.hip - multi-query attention for long query runs (chunked prefill,
// "vLLM 推理引擎源码级拆解" §6.3) on 32 x 32 matrix-core tiles, with the K/V
// of a stage staged in LDS and shared by the waves of a workgroup.
//
// What is computed is that of multi_query.hip: query token i of sequence s
// sits at position L - Qn + i and attends to tokens 0 .. L - Qn + i through
// the block table; a token whose position is negative gets a zero row.
//
// Work layout.
//   - A workgroup serves one (sequence, KV head) and 128 / G consecutive
//     query tokens; each of its 4 waves owns 32 query rows, the (token,
//     head) pairs of 32 / G tokens (GQA: the G heads of a token share the
//     KV head, so every K/V byte a wave reads feeds G rows).
//   - The context the workgroup's last token sees is walked in stages of 64
//     keys.  A stage's K and V rows (through the block table; rows past the
//     context read zeros) go to one of two LDS buffers, one barrier per
//     stage; the next stage's rows are in flight during the current stage's
//     arithmetic.  K is loaded straight into LDS by buffer loads with the
//     LDS as destination (unpadded rows, 16-byte units XOR-swizzled by row);
//     V passes through registers and is stored transposed (one LDS row per
//     dimension d, the stage's keys along it), so that each lane's value
//     operand of the PV product is one 16-byte LDS read.
//   - Stages all of whose keys every row of a wave sees run in a loop
//     without the causal mask, the rest in a second loop with it.
//   - (Sequence, KV head) pairs are dealt to the XCDs round robin, all the
//     groups of a pair on one XCD, longest contexts first.
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
//     {4g..4g+3, 8+4g..8+4g+3} of each 16-key step; the V^T rows keep each
//     16-key group's quads in the order (0, 2, 1, 3), so those 8 keys are
//     16 contiguous bytes.
//   Every value of a lane's accumulators belongs to its own query row, so
//   the softmax's rescale is a per-lane multiply; the row's max and sum
//   combine the two lanes of a row (l and l ^ 32) with one lane swap.
//
// Softmax: base-2 scores (scale * log2 e folded), lazy rescale (the
// reference max moves only when exceeded by more than 8), weights fed to
// the PV product as bf16 hi + lo (~16 significant bits) for bf16 queries
// and as f16 for f16 queries, so the only 8-bit rounding left is the stored
// output.  Causal masking is applied only on the sub-tiles that reach past
// the first position any of the wave's rows sees.
#include "tile_mfma.hpp"

namespace pkv {
namespace {

using namespace mfma;

typedef float f32x16 __attribute__((ext_vector_type(16)));

template <class Q>
struct Mma32;
template <>
struct Mma32<BF16> {
    typedef __bf16 T;
    typedef bf16x8 v8;
    static constexpr bool kSplitP = true;
    __device__ static inline f32x16 mma(v8 a, v8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};
template <>
struct Mma32<F16> {
    typedef _Float16 T;
    typedef f16x8 v8;
    static constexpr bool kSplitP = false;
    __device__ static inline f32x16 mma(v8 a, v8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};

constexpr int kWaves = 4;
constexpr int kRows = 32;     // query rows per wave
constexpr int kStage = 64;    // keys per LDS stage
constexpr int kSub = 32;      // keys per matrix-core sub-tile

template <int D>
struct Shape {
    static constexpr int kRow = 2 * D;                 // bytes of one head's K or V row
    static constexpr int kK = kStage * kRow;           // K of a stage (rows swizzled, unpadded)
    static constexpr int kVStride = 2 * kStage + 16;   // V^T rows (one per d), padded
    static constexpr int kV = D * kVStride;            // V^T of a stage
    static constexpr int kBuf = kK + kV;
    static constexpr int kLds = 2 * kBuf;              // double buffer
    static constexpr int kChunks = kRow / 16;          // 16-byte pieces of a row
    // keys of one wave-wide 16-byte load (64 lanes): 4 at D = 128, 8 at D = 64
    static constexpr int kKpl = 64 / kChunks;
    // V rows each thread moves per stage (one 16-byte piece of each, the
    // same piece): 4 at D = 128, 2 at D = 64
    static constexpr int kKpt = kStage * kChunks / (64 * kWaves);
    static constexpr int kQS = D / 16;                 // QK instructions (16 d each)
    static constexpr int kNT = D / 32;                 // output tiles of 32 d
    static_assert(kKpt * 64 * kWaves == kStage * kChunks, "stage split");
    static_assert(kKpt == 2 || kKpt == 4, "a thread's keys lie in one quad");
};

// Two 16-bit values, lo from a and hi from b, taken from the same half of
// two dwords: half 0 the low halves, half 1 the high halves.
__device__ inline uint32_t pair16(uint32_t a, uint32_t b, int half) {
    return half ? (a >> 16) | (b & 0xFFFF0000u) : (a & 0xFFFFu) | (b << 16);
}

// Byte offset, among a V^T row's 128 key bytes, of key k of a stage.  Each
// 16-key group is 32 bytes, 16 per lane half g of the value operand, which
// takes keys {4g..4g+3, 8+4g..8+4g+3}; they are stored in the order
// (4g, 4g+1, 8+4g, 9+4g, 4g+2, 4g+3, 10+4g, 11+4g), so that the two key
// pairs (2j, 2j+1) and (8+2j, 9+2j) a thread moves are 8 adjacent bytes.
// The weights are packed into the other operand in the same order.
__device__ inline uint32_t vt_key(int k) {
    const int kk = k & 15, w = kk & 3;
    const int e = (w >> 1) * 4 + (kk >> 3) * 2 + (w & 1);
    return (uint32_t)((k >> 4) * 32 + ((kk >> 2) & 1) * 16 + e * 2);
}

// K rows of a stage buffer are unpadded, their 16-byte units XORed with
// row % KSW (the units per row, at most 16), so that the rows a score read
// takes at once fall in distinct banks.
template <int ROW>
constexpr int k_swizzle() { return ROW / 16 < 16 ? ROW / 16 : 16; }

// Byte address of key byte `kb` of V^T row `row` in a stage buffer.  The
// 16-byte unit is XORed with (row / 8) % 8: the stores of a wave write rows
// 8 apart (which would all fall in one bank), the value reads of a wave read
// 8 consecutive rows with one XOR (the row padding keeps those apart).
template <int STRIDE>
__device__ inline uint32_t vt_addr(int row, uint32_t kb) {
    return (uint32_t)row * STRIDE + ((((kb >> 4) ^ ((uint32_t)row >> 3)) & 7u) << 4) + (kb & 15u);
}

// PAIR: 8-token blocks, so the 16 keys a wave loads span two blocks.
template <class Q, int D, bool PAIR>
__global__ __launch_bounds__(64 * kWaves, 2) void prefill_kernel(DecodeParams p) {
    typedef Shape<D> SH;
    typedef Mma32<Q> M;
    typedef typename M::T T;
    typedef typename M::v8 v8;
    extern __shared__ __attribute__((aligned(16))) char lds[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int c = lane & 31;               // this lane's query row within the wave
    const int g = lane >> 5;               // lane half
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    // workgroup -> (sequence, KV head, group of query tokens).  Workgroups
    // are dealt to the XCDs in turn (blockIdx % 8).  The (sequence, KV head)
    // pairs are dealt to the XCDs round robin, so each XCD gets a share of
    // every sequence's work, and all the groups of a pair run on one XCD,
    // sharing its L2.  Each XCD takes the groups reading the longest
    // contexts (the last query tokens) of all its pairs first.
    const int G = p.G;
    const int tpw = kRows / G;             // query tokens per wave
    const int tpg = kWaves * tpw;          // per workgroup
    const int pairs = p.S * p.Hkv;
    const int per_xcd = (pairs + 7) / 8;   // pairs per XCD (the last ones short)
    const int xcd = (int)(blockIdx.x % 8);
    const int j = (int)(blockIdx.x / 8);
    const int pair = (j % per_xcd) * 8 + xcd;
    const int grp = p.max_groups - 1 - j / per_xcd;
    if (pair >= pairs || grp < 0) return;  // whole workgroup
    const int h = pair % p.Hkv;
    const int s = pair / p.Hkv;
    const int q0 = __builtin_amdgcn_readfirstlane(p.q_start[s]);
    const int Qn = __builtin_amdgcn_readfirstlane(p.q_start[s + 1]) - q0;
    const int wg_base = grp * tpg;
    if (wg_base >= Qn) return;             // whole workgroup
    int L = __builtin_amdgcn_readfirstlane(p.lens[s]);
    L = L < p.len_cap ? L : p.len_cap;
    // keys the workgroup's last query token sees (0: none)
    const int wg_end = max(0, L - Qn + min(wg_base + tpg, Qn));

    // ---- this lane's query row ----
    const int tok = wg_base + wave * tpw + c / G;   // query token within the sequence
    const int hh = c % G;
    const bool has_row = tok < Qn;
    const int pos = L - Qn + tok;                   // its position in the sequence
    const bool sees = has_row && pos >= 0;
    // last key this row sees; rows that see nothing read everything (zero
    // queries, never written), which keeps every row's max finite
    const int lim = sees ? pos : INT_MAX;
    // Scores enter the exponent as fma(s, |scale'|, -m); a negative scale is
    // carried by the query's sign (exact).
    const float sl2 = p.scale_log2;
    const float sla = fabsf(sl2);
    v8 qf[SH::kQS];
    {
        const T* qrow = (const T*)p.q + ((size_t)(q0 + (sees ? tok : 0)) * p.Hq +
                                         (size_t)h * G + hh) * D;
        const uint32_t flip = sl2 < 0.0f ? 0x80008000u : 0u;
#pragma unroll
        for (int i = 0; i < SH::kQS; i++) {
            u32x4 x = sees ? *(const u32x4*)(qrow + (D / 2) * g + 8 * i) : u32x4{};
            x ^= flip;
            qf[i] = __builtin_bit_cast(v8, x);
        }
    }
    // wave-uniform bounds over the rows that see keys: the last key any of
    // them sees, and the last key all of them see
    int wlast = sees ? pos : -1;
    int wvis = sees ? pos : INT_MAX;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        wlast = max(wlast, __shfl_xor(wlast, o, 64));
        wvis = min(wvis, __shfl_xor(wvis, o, 64));
    }
    wlast = __builtin_amdgcn_readfirstlane(wlast);
    wvis = __builtin_amdgcn_readfirstlane(wvis);

    // ---- stage loads ----
    // A wave moves the 16 consecutive, aligned keys 16 wave .. of a stage:
    // one block, or two 8-token blocks (PAIR), whose table entries are
    // wave-uniform, so every load has a scalar buffer descriptor.  Rows at
    // or past wg_end take an out-of-range offset and read zeros.
    //   K goes straight to LDS (buffer loads with the LDS as destination):
    //   load r of the wave covers keys 16 wave + kKpl r .. + kKpl - 1 (one
    //   block), lane i writing 16 bytes at i * 16 from the load's first row,
    //   i.e. row i / kChunks, swizzled unit i % kChunks, which holds unit
    //   (i % kChunks) ^ (row % 8) of the key's row.
    //   V passes through registers to be transposed: thread (j = lane /
    //   kChunks, ch = lane % kChunks) moves piece ch of the keys 2j, 2j+1
    //   and, at head_dim 128, 8+2j, 9+2j of the wave's 16 (load r takes key
    //   8 (r / 2) + 2j + r % 2, one block per load at head_dim 128).
    const int bs_shift = p.bs == 8 ? 3 : (p.bs == 16 ? 4 : 5);
    const uint32_t pool_row = (uint32_t)p.Hkv * SH::kRow;       // bytes between slots
    const uint32_t blk_bytes = (uint32_t)p.bs * pool_row;
    const uint32_t head_off = (uint32_t)h * SH::kRow;
    const int lj = lane / SH::kChunks;
    const int ch = lane % SH::kChunks;
    const int last_blk = wg_end > 0 ? (wg_end - 1) >> bs_shift : 0;
    // the sequence's live table entries, read with buffer loads (a vector
    // memory access, so waiting for one never waits for LDS traffic)
    const rsrc_t tbl = make_rsrc((const char*)(p.tables + (size_t)s * p.max_blocks),
                                 (uint32_t)(last_blk + 1) * 4u);
    // table entries of the wave's blocks in stage st (requested one stage
    // before they are used)
    auto entry = [&](int st, int second) {
        const int b = min(((st * kStage + 16 * wave) >> bs_shift) + second, last_blk);
        return (int)Buf<4>::load(tbl, (uint32_t)b * 4u);
    };
    auto blk = [&](int e) {
        const uint32_t b = (uint32_t)__builtin_amdgcn_readfirstlane(e);
        return b < (uint32_t)p.NB ? b : (uint32_t)p.NB - 1u;
    };
    // in-block byte offset of key t (a key of this stage), or out of range
    auto row_off = [&](int t) {
        return t < wg_end ? (uint32_t)(t & (p.bs - 1)) * pool_row + head_off : kOOB;
    };
    constexpr int kVL = SH::kKpt;          // V loads per thread per stage
    u32x4 vr[kVL];
    auto load_stage = [&](int st, int ea, int eb, int buf) {
        const uint32_t ba = blk(ea);
        const uint32_t bb = PAIR ? blk(eb) : ba;
        const rsrc_t rka = make_rsrc((const char*)p.k + (size_t)ba * blk_bytes, blk_bytes);
        const rsrc_t rkb = make_rsrc((const char*)p.k + (size_t)bb * blk_bytes, blk_bytes);
        const rsrc_t rva = make_rsrc((const char*)p.v + (size_t)ba * blk_bytes, blk_bytes);
        const rsrc_t rvb = make_rsrc((const char*)p.v + (size_t)bb * blk_bytes, blk_bytes);
        const int t0 = st * kStage + 16 * wave;
        char* kdst = lds + buf * SH::kBuf + 16 * wave * SH::kRow;
#pragma unroll
        for (int r = 0; r < 16 / SH::kKpl; r++) {
            const int row = r * SH::kKpl + lj;         // within the wave's 16
            const uint32_t u = (uint32_t)(ch ^ (row & (k_swizzle<SH::kRow>() - 1)));
            const uint32_t off = row_off(t0 + row);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                PAIR && row >= 8 ? rkb : rka,
                (__attribute__((address_space(3))) void*)(kdst + r * SH::kKpl * SH::kRow), 16,
                off == kOOB ? kOOB : off + 16u * u, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < kVL; r++) {
            if constexpr (SH::kKpt == 4) {
                const int row = 8 * (r >> 1) + 2 * lj + (r & 1);
                const uint32_t off = row_off(t0 + row);
                vr[r] = Buf<16>::load(PAIR && r >= 2 ? rvb : rva,
                                      off == kOOB ? kOOB : off + 16u * (uint32_t)ch);
            } else {
                // head_dim 64: keys 2j, 2j+1, j < 8, across both 8-token halves
                const int row = 2 * lj + r;
                const uint32_t off = row_off(t0 + row);
                const uint32_t o = off == kOOB ? kOOB : off + 16u * (uint32_t)ch;
                if constexpr (PAIR) {
                    const bool second = row >= 8;
                    vr[r] = Buf<16>::load(rva, second ? kOOB : o) |
                            Buf<16>::load(rvb, second ? o : kOOB);
                } else {
                    vr[r] = Buf<16>::load(rva, o);
                }
            }
        }
    };
    auto store_stage = [&](int buf) {
        char* vb = lds + buf * SH::kBuf + SH::kK;
        // V^T: dimension 8 ch + d, this thread's keys side by side
        const uint32_t kofs = vt_key(16 * wave + 2 * lj);
#pragma unroll
        for (int d = 0; d < 8; d++) {
            char* at = vb + vt_addr<SH::kVStride>(8 * ch + d, kofs);
            const int w = d >> 1, half = d & 1;
            if constexpr (SH::kKpt == 4) {
                u32x2 x;
                x[0] = pair16(vr[0][w], vr[1][w], half);
                x[1] = pair16(vr[2][w], vr[3][w], half);
                *(u32x2*)at = x;
            } else {
                *(uint32_t*)at = pair16(vr[0][w], vr[1][w], half);
            }
        }
    };

    // ---- running state of this lane's row ----
    f32x16 o[SH::kNT];
#pragma unroll
    for (int n = 0; n < SH::kNT; n++) o[n] = f32x16{};
    float m = -INFINITY, l = 0.0f;   // reference max (scaled, base 2) and sum

    // Lane-constant LDS addresses of the operand reads, relative to a stage
    // buffer.  K: row c of a sub-tile, unit (D / 16) g + i of the score
    // step i, swizzled.  V^T: row c of output tile 0, the lane half's 16
    // bytes of 16-key step ii of sub-tile 0; the unit swizzle (row / 8) % 8
    // splits into these lane bits (0-1) and a bit 2 that depends only on
    // the tile n and the sub-tile, which the reads add as a constant.
    uint32_t ka[SH::kQS], va[2];
#pragma unroll
    for (int i = 0; i < SH::kQS; i++)
        ka[i] = (uint32_t)(c * SH::kRow) +
                (uint32_t)((((D / 16) * g + i) ^ (c & (k_swizzle<SH::kRow>() - 1))) << 4);
#pragma unroll
    for (int ii = 0; ii < 2; ii++)
        va[ii] = (uint32_t)(SH::kK + c * SH::kVStride) +
                 (uint32_t)((((2 * ii + g) ^ (c >> 3)) & 3) << 4);

    // One 32-key sub-tile u of the stage in LDS buffer `base`: scores, the
    // softmax update, the value products.
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    auto sub_tile = [&](const char* base, int u, int kb, auto mask) {
        constexpr bool MASK = decltype(mask)::value;
        // all K fragments requested before the first product
        v8 kf[SH::kQS];
#pragma unroll
        for (int i = 0; i < SH::kQS; i++)
            kf[i] = *(const v8*)(base + ka[i] + u * kSub * SH::kRow);
        f32x16 sc = f32x16{};
#pragma unroll
        for (int i = 0; i < SH::kQS; i++) sc = M::mma(kf[i], qf[i], sc);
        // the value fragments, in flight during the softmax
        v8 vf[2][SH::kNT];
#pragma unroll
        for (int ii = 0; ii < 2; ii++)
#pragma unroll
            for (int n = 0; n < SH::kNT; n++)
                vf[ii][n] = *(const v8*)(base + va[ii] + 32 * n * SH::kVStride +
                                         64 * ((u ^ n) & 1));

        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; r++) {
            const int key = kb + 8 * (r >> 2) + 4 * g + (r & 3);
            mx = fmaxf(mx, (!MASK || key <= lim) ? sc[r] : -INFINITY);
        }
        mx = swap_max32(mx);
        const float mxs = mx == -INFINITY ? -INFINITY : mx * sla;
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
        float ls = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; r++) {
            const float e = __builtin_amdgcn_exp2f(fmaf(sc[r], sla, nm));
            const int key = kb + 8 * (r >> 2) + 4 * g + (r & 3);
            pz[r] = (!MASK || key <= lim) ? e : 0.0f;
            ls += pz[r];
        }
        l += ls;
#pragma unroll
        for (int ii = 0; ii < 2; ii++) {
            // element e of the operand is score register kPerm[e] of the
            // 16-key step (the V^T key order above); pairs (2q, 2q+1)
            constexpr int kPerm[8] = {0, 1, 4, 5, 2, 3, 6, 7};
            uint32_t hw[4], lw[4];
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const f32x2 x = {pz[8 * ii + kPerm[2 * q]], pz[8 * ii + kPerm[2 * q + 1]]};
                if constexpr (M::kSplitP) {
                    hw[q] = __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
                    const f32x2 h = {__builtin_bit_cast(float, hw[q] << 16),
                                     __builtin_bit_cast(float, hw[q] & 0xFFFF0000u)};
                    lw[q] = __builtin_bit_cast(uint32_t, __builtin_convertvector(x - h, bf16x2));
                } else {
                    hw[q] = __builtin_bit_cast(uint32_t, __builtin_convertvector(x, f16x2));
                }
            }
            const v8 hi = __builtin_bit_cast(v8, u32x4{hw[0], hw[1], hw[2], hw[3]});
#pragma unroll
            for (int n = 0; n < SH::kNT; n++) o[n] = M::mma(vf[ii][n], hi, o[n]);
            if constexpr (M::kSplitP) {
                const v8 lo = __builtin_bit_cast(v8, u32x4{lw[0], lw[1], lw[2], lw[3]});
#pragma unroll
                for (int n = 0; n < SH::kNT; n++) o[n] = M::mma(vf[ii][n], lo, o[n]);
            }
        }
    };

    const int nstage = (wg_end + kStage - 1) / kStage;
    int ea = 0, eb = 0;
    if (nstage > 0) {
        load_stage(0, entry(0, 0), PAIR ? entry(0, 1) : 0, 0);
        ea = entry(1, 0);
        if constexpr (PAIR) eb = entry(1, 1);
        store_stage(0);
    }
    __syncthreads();
    // Stages [st0, st1), every sub-tile with the causal limits (MASK) or,
    // for stages all of whose keys every row of the wave sees, without.
    // The two kinds run in two loops rather than behind a branch in one, so
    // each keeps one register assignment; every stage passes one barrier,
    // so waves that split the stages differently still meet at each one.
    auto run_stages = [&](int st0, int st1, auto mask) {
        for (int st = st0; st < st1; st++) {
            const int buf = st & 1;
            // next stage's rows in flight during this stage's arithmetic
            // (past the end they are all out of range and touch nothing; K
            // lands in the other buffer, which no wave reads until the next
            // barrier)
            load_stage(st + 1, ea, eb, buf ^ 1);
            ea = entry(st + 2, 0);
            if constexpr (PAIR) eb = entry(st + 2, 1);
            const char* base = lds + buf * SH::kBuf;
#pragma unroll
            for (int u = 0; u < kStage / kSub; u++) {
                const int kb = st * kStage + u * kSub;
                if (kb <= wlast) sub_tile(base, u, kb, mask);            // wave-uniform
            }
            store_stage(buf ^ 1);                  // read by no wave since the last barrier
            __syncthreads();
        }
    };
    // stage st is seen whole by every row of the wave when st * kStage +
    // kStage - 1 <= wvis (wvis is INT_MAX for a wave without rows: it
    // computes nothing and only passes the barriers)
    const int nfull = (int)min64(nstage, ((int64_t)wvis + 1) / kStage);
    run_stages(0, nfull, std::false_type{});
    run_stages(nfull, nstage, std::true_type{});

    // ---- epilogue: normalise and store this lane's row ----
    if (has_row) {
        const float l_tot = swap_sum32(l);
        const float inv = sees && l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
        T* orow = (T*)p.out + ((size_t)(q0 + tok) * p.Hq + (size_t)h * G + hh) * D;
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
}

template <class Q, int D>
hipError_t launch_dd(const DecodeParams& p, hipStream_t st) {
    typedef Shape<D> SH;
    const long pairs = (long)p.S * p.Hkv;
    const long wgs = (pairs + 7) / 8 * 8 * p.max_groups;   // per_xcd pairs x groups, x 8
    void* args[] = {const_cast<DecodeParams*>(&p)};
    const void* k = p.bs == 8 ? reinterpret_cast<const void*>(prefill_kernel<Q, D, true>)
                              : reinterpret_cast<const void*>(prefill_kernel<Q, D, false>);
    return hipLaunchKernel(k, dim3((unsigned)wgs), dim3(64 * kWaves), args, SH::kLds, st);
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
