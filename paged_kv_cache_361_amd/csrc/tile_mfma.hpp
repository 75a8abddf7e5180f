// tile_mfma.hpp - the matrix-core tile of paged decode attention, shared by
// the per-unit kernel (decode_mfma.hip) and the balanced persistent kernel
// (decode_balanced.hip).
//
// One wavefront serves the G <= 16 query heads of one KV head, 16 tokens at
// a time ("vLLM 推理引擎源码级拆解" §2.3: single-query attention through the block
// table with a running max / running sum softmax):
//
//   scores  S^T[token][head] = K_tile[16 x D] * Q^T[D x 16]
//           v_mfma_f32_16x16x32_{bf16,f16}: A = K rows (lane%16 = token, the
//           lane's 8 contraction elements are a 16-byte slice of the row), B =
//           the query heads (lane%16 = head, zero past G).  The result lands
//           with lane%16 = head and register r = token 4*(lane/16) + r.
//   output  O[head][d] += P[head][token] * V_tile[16 x D]
//           v_mfma_f32_16x16x16_{bf16,f16}, one per 16 output columns.  The
//           score layout above is exactly the A layout of this instruction
//           (lane%16 = head, 4 consecutive tokens per lane), so the softmax
//           weights feed it without any data movement.  For B each lane loads
//           the rows of its 4 tokens restricted to 8 contiguous columns and the
//           columns are assigned as d = 8*(lane%16) + n for tile n, which turns
//           the transpose the instruction needs into register permutes.
//
// Memory side.  Every K/V access is a non-temporal buffer load whose 128-bit descriptor
// holds the 64-bit base of one physical block (plus the head offset) in
// scalar registers, with 32-bit per-lane offsets inside the block.  Rows past
// the end of a sequence get an offset beyond the descriptor's range: the
// hardware returns zeros without touching memory, so masked tokens cost no
// bandwidth and whatever the pool holds there (NaN poison included) never
// reaches the arithmetic.  Block ids come from a 64-entry window of the block
// table held one entry per lane and broadcast with readlane.
//
// Softmax bookkeeping.  Scores are kept in base-2 units (log2(e) and the
// scale folded into one multiplier).  The running reference maximum of a
// head is raised only when a tile's maximum exceeds it by more than kTau, so
// the accumulator rescale is rare; weights are then bounded by 2^kTau, which
// fp32 sums absorb without loss.
//
// E4M3 caches are widened to the query's 16-bit type with the gfx950 packed
// conversion (exact: every E4M3 value is a bf16 and an f16 value); the K and
// V scales are folded into the score scale and the output scale.
//
// With a bf16 query the softmax weights are fed as a bf16 pair hi + lo
// (hi = bf16(p), lo = bf16(p - hi)), i.e. ~16 significant bits, so the only
// 8-bit rounding left in the kernel is the stored output itself.
#pragma once

#include <cfloat>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace pkv {
namespace mfma {

constexpr float kTau = 8.0f;            // lazy-rescale threshold (base-2 units)
constexpr uint32_t kOOB = 0x80000000u;  // past any descriptor range: reads 0
// Cache policy of the K/V loads: non-temporal.  Every K/V byte is read once
// per call, so keeping it out of the caches' replacement costs nothing, and
// on MI355X random 4 KiB block slices stream about 14% faster this way
// (6.9 against 6.06 TB/s in a read-only probe of the same pattern).
constexpr int kStream = 2;

typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef __attribute__((address_space(3))) char lds_t;

// s_waitcnt on the vector-memory count alone (expcnt and lgkmcnt at their
// maxima): returns once at most N vector-memory instructions of the wave
// are still in flight.  The count field is 6 bits, split low 4 / high 2.
template <int N>
__device__ inline void vm_wait() {
    static_assert(N >= 0 && N < 64, "vmcnt field");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0xF70);
}

// A 16-byte LDS read through a restrict pointer: the compiler then does not
// treat it as possibly reading what an LDS-direct load still in flight
// writes, and adds no wait of its own for those loads.
__device__ inline u32x4 lds_read16(const lds_t* __restrict__ p) {
    return *(const __attribute__((address_space(3))) u32x4*)p;
}

// Raw buffer descriptor over [base, base + bytes): stride 0, 32-bit format
// word of the gfx9 family.
__device__ inline rsrc_t make_rsrc(const char* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), 0, (int)bytes,
                                             0x00020000);
}

template <int BYTES>
struct Buf;
template <>
struct Buf<16> {
    typedef u32x4 T;
    __device__ static inline T load(rsrc_t r, uint32_t off) {
        return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
    }
    __device__ static inline T stream(rsrc_t r, uint32_t off) {
        return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kStream));
    }
};
template <>
struct Buf<8> {
    typedef u32x2 T;
    __device__ static inline T load(rsrc_t r, uint32_t off) {
        return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0));
    }
    __device__ static inline T stream(rsrc_t r, uint32_t off) {
        return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, kStream));
    }
};
template <>
struct Buf<4> {
    typedef uint32_t T;
    __device__ static inline T load(rsrc_t r, uint32_t off) {
        return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
    }
    __device__ static inline T stream(rsrc_t r, uint32_t off) {
        return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, kStream);
    }
};

template <class Q>
struct Mfma;

template <>
struct Mfma<BF16> {
    typedef __bf16 T;
    typedef bf16x8 v8;
    typedef bf16x4 v4;
    static constexpr bool kSplitP = true;
    __device__ static inline f32x4 qk(v8 a, v8 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    __device__ static inline f32x4 pv(v4 a, v4 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
    }
    // 4 E4M3 codes (one dword) -> 4 bf16.
    __device__ static inline v4 from_fp8x4(uint32_t w) {
        const auto lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
        const auto hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
        return v4{lo[0], lo[1], hi[0], hi[1]};
    }
};

template <>
struct Mfma<F16> {
    typedef _Float16 T;
    typedef f16x8 v8;
    typedef f16x4 v4;
    static constexpr bool kSplitP = false;
    __device__ static inline f32x4 qk(v8 a, v8 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
    __device__ static inline f32x4 pv(v4 a, v4 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
    }
    __device__ static inline v4 from_fp8x4(uint32_t w) {
        typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
        const f16x2 lo = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
        const f16x2 hi = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true));
        return v4{lo[0], lo[1], hi[0], hi[1]};
    }
};

// Wave-uniform addressing of one KV head's rows in the pool.
struct Head {
    const char* kbase;     // k_cache + head offset
    const char* vbase;     // v_cache + head offset
    uint32_t row_bytes;    // bytes between consecutive slots
    uint32_t blk_bytes;    // bytes per block
    uint32_t rec_bytes;    // descriptor range from a block base
    uint32_t nb_last;      // last valid block id
    int bs_shift;          // log2(block_size)
};

template <class C, int D>
__device__ inline Head make_head(const DecodeParams& p, int h) {
    constexpr int EB = C::kBytes;
    Head hd;
    const uint32_t head_off = (uint32_t)(h * D * EB);
    hd.row_bytes = (uint32_t)(p.Hkv * D * EB);
    hd.blk_bytes = (uint32_t)p.bs * hd.row_bytes;
    hd.rec_bytes = hd.blk_bytes - head_off;
    hd.kbase = (const char*)p.k + head_off;
    hd.vbase = (const char*)p.v + head_off;
    hd.nb_last = (uint32_t)p.NB - 1u;
    hd.bs_shift = p.bs == 8 ? 3 : (p.bs == 16 ? 4 : 5);
    return hd;
}

// PAIR: block size 8, so a 16-token tile spans two blocks.
// KLDS: the K tile goes from memory straight into LDS, row by row
// (buffer_load ... lds), and is read back in the operand layout (see
// issue_as and consume); otherwise K rows load into registers directly in the
// operand layout.  Row-order loads cover 4 rows x 256 bytes per instruction
// where the operand layout covers 16 rows x 64 bytes, and on MI355X a read
// probe of the decode's own tiles streamed the 40-head pool (10 KiB between
// a head's rows) 16% faster that way, and the 8-head pool 4% faster.
template <class Q, class C, int D, bool PAIR, bool KLDS = false>
struct TileMath {
    typedef Mfma<Q> M;
    typedef typename M::T T;
    typedef typename M::v8 v8;
    typedef typename M::v4 v4;
    static constexpr bool kFp8 = std::is_same<C, FP8>::value;
    static constexpr int EB = C::kBytes;           // cache bytes per element
    static constexpr int KS = D / 32;              // QK contraction steps
    static constexpr int NT = D / 16;              // PV column tiles = columns per lane
    static constexpr int KL = kFp8 ? D / 64 : KS;  // 16-byte K loads per lane per tile
    static constexpr int VB = NT * EB;             // bytes of one V row slice per lane
    typedef T vrow __attribute__((ext_vector_type(NT)));
    typedef typename Buf<VB>::T vraw;
    // LDS-staged K: 16-byte pieces per row, rows per load instruction, and
    // the bytes of one tile's 16 rows
    static constexpr int KR = D * EB / 16;
    static constexpr int kRowsPerLoad = 64 / KR;
    static constexpr int kKSlot = 16 * 16 * KR;
    static_assert(KL * 1024 == kKSlot, "a tile's K is KL loads of 1 KiB");
    // a load of an LDS-staged two-block tile must lie in one block
    static_assert(!(KLDS && PAIR) || kRowsPerLoad <= 8, "LDS-direct loads within one block");
    // vector-memory instructions issue() makes per tile
    static constexpr int kLoadsPerTile = (KLDS ? KL : (PAIR ? 2 : 1) * KL) + (PAIR ? 8 : 4);

    struct TileRegs {
        u32x4 k[KL];
        vraw v[4];
    };
    struct TileLds {
        vraw v[4];
    };
    typedef std::conditional_t<KLDS, TileLds, TileRegs> Tile;

    // Piece p of K row r is stored at piece p ^ kswz(r) of the row's LDS
    // slot, so that the 16 rows one operand read touches (one piece each)
    // fall on distinct banks: r % 16 for rows of 16 or more pieces, r / 2 % 8
    // for 8 pieces (two rows per 64 banks), r / 4 % 4 for 4 pieces.
    __device__ static inline int kswz(int r) {
        if constexpr (KR >= 16) return r & 15;
        else if constexpr (KR == 8) return (r >> 1) & 7;
        else return (r >> 2) & 3;
    }
    // Running state of one (sequence piece, KV head): reference max and this
    // lane's share of the sum for head lane%16, accumulator rows 4*(lane/16)+r.
    struct Acc {
        f32x4 o[NT];
        float m;
        float l;
    };

    int lane, g4, j16;
    uint32_t kcol[KL];     // lane-constant byte offsets inside a slot row
    uint32_t vcol;
    // KLDS: row of load i this lane fills and the byte offset of its piece
    // in that row; byte offset of operand piece i in the tile's LDS slot
    int kdr[KLDS ? KL : 1];
    uint32_t kdp[KLDS ? KL : 1], krd[KLDS ? KL : 1];

    __device__ TileMath() {
        lane = threadIdx.x & 63;
        g4 = lane >> 4;
        j16 = lane & 15;
#pragma unroll
        for (int i = 0; i < KL; i++)
            kcol[i] = kFp8 ? (uint32_t)(64 * i + 16 * g4) : (uint32_t)((32 * i + 8 * g4) * EB);
        vcol = (uint32_t)(NT * j16 * EB);
        if constexpr (KLDS) {
#pragma unroll
            for (int i = 0; i < KL; i++) {
                // load i fills rows kRowsPerLoad i .. with lane-consecutive
                // 16-byte LDS slots: lane -> (row, slot piece lane % KR)
                kdr[i] = kRowsPerLoad * i + lane / KR;
                kdp[i] = 16u * (uint32_t)((lane % KR) ^ kswz(kdr[i]));
                // the operand wants piece kcol[i] / 16 of row j16
                krd[i] = (uint32_t)(j16 * 16 * KR) + 16u * (uint32_t)(((int)kcol[i] / 16) ^ kswz(j16));
            }
        }
    }

    // Query heads of the group as the B operand of the score product; `q`
    // is row 0 of the group ([G][D]), heads past G read as zeros.
    __device__ inline void load_q(const T* q, int G, v8 (&qb)[KS]) const {
        const T* qrow = q + (size_t)j16 * D;
#pragma unroll
        for (int kk = 0; kk < KS; kk++) {
            const int d0 = kFp8 ? (kk >> 1) * 64 + 16 * g4 + (kk & 1) * 8 : 32 * kk + 8 * g4;
            if (j16 < G) qb[kk] = *(const v8*)(qrow + d0);
            else qb[kk] = v8{};
        }
    }

    __device__ inline void reset(Acc& a) const {
#pragma unroll
        for (int n = 0; n < NT; n++) a.o[n] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        // below every score, but finite: a column that has seen nothing
        // yet (masked rows score -inf) gets weights exp2(-inf - m) = 0, not
        // the NaN of -inf - -inf
        a.m = -FLT_MAX;
        a.l = 0.0f;
    }

    // Issues the loads of the 16-token tile starting at token t0 (no wait).
    // lim = index within the tile of its last live row (< 0: the whole tile
    // is dead and reads zeros).  Block ids come from `win`, the table entries
    // from block wb on (t0's block and, with PAIR, the next one must lie in
    // the window when live).
    __device__ inline void issue(const Head& hd, int t0, int lim, int wb, int win,
                                 Tile& tl, lds_t* kslot = nullptr) const {
        issue_as<PAIR>(hd, t0, lim, wb, win, tl, kslot);
    }

    // issue() for 8-token blocks (PR) or larger ones, whatever the tile's
    // own PAIR: a kernel whose wavefronts meet both block sizes picks per
    // wavefront.
    // KLDS: kslot (wave-uniform) receives the tile's K rows, kKSlot bytes;
    // rows past lim are written as zeros.  The caller waits for the loads
    // (vm_wait) before consume() reads them.
    template <bool PR>
    __device__ inline void issue_as(const Head& hd, int t0, int lim, int wb, int win,
                                    Tile& tl, lds_t* kslot = nullptr) const {
        uint32_t pa = 0, pb = 0;
        if (lim >= 0) {
            const int blk = (t0 >> hd.bs_shift) - wb;
            pa = (uint32_t)__builtin_amdgcn_readlane(win, blk);
            pa = pa < hd.nb_last ? pa : hd.nb_last;
            if (PR && lim >= 8) {
                pb = (uint32_t)__builtin_amdgcn_readlane(win, blk + 1);
                pb = pb < hd.nb_last ? pb : hd.nb_last;
            }
        }
        const rsrc_t ka = make_rsrc(hd.kbase + (size_t)pa * hd.blk_bytes, hd.rec_bytes);
        const rsrc_t va = make_rsrc(hd.vbase + (size_t)pa * hd.blk_bytes, hd.rec_bytes);
        if constexpr (KLDS && PR) {
            static_assert(PAIR, "the ring's tiles are counted as two-block ones");
            // 8-token blocks: the tile starts a block, rows 0-7 lie in block
            // a and rows 8-15 in block b, and each row-order load covers
            // rows of one block only
            const rsrc_t kb = make_rsrc(hd.kbase + (size_t)pb * hd.blk_bytes, hd.rec_bytes);
            const rsrc_t vb = make_rsrc(hd.vbase + (size_t)pb * hd.blk_bytes, hd.rec_bytes);
#pragma unroll
            for (int i = 0; i < KL; i++) {
                const uint32_t off =
                    kdr[i] <= lim ? (uint32_t)(kdr[i] & 7) * hd.row_bytes + kdp[i] : kOOB;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(kRowsPerLoad * i >= 8 ? kb : ka,
                                                         (lds_t*)(kslot + 1024 * i), 16, off, 0, 0,
                                                         kStream);
            }
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int tv = 4 * g4 + r;
                const uint32_t vo = (uint32_t)(tv & 7) * hd.row_bytes;
                const uint32_t voa = tv <= lim && tv < 8 ? vo : kOOB;
                const uint32_t vob = tv <= lim && tv >= 8 ? vo : kOOB;
                tl.v[r] = Buf<VB>::stream(va, voa + vcol) | Buf<VB>::stream(vb, vob + vcol);
            }
        } else if constexpr (KLDS) {
            static_assert(!PAIR, "the ring's tiles are counted as one-block ones");
            const uint32_t in_blk = (uint32_t)(t0 & ((1 << hd.bs_shift) - 1));
#pragma unroll
            for (int i = 0; i < KL; i++) {
                const uint32_t off =
                    kdr[i] <= lim ? (in_blk + (uint32_t)kdr[i]) * hd.row_bytes + kdp[i] : kOOB;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(ka, (lds_t*)(kslot + 1024 * i), 16, off, 0, 0,
                                                         kStream);
            }
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int tv = 4 * g4 + r;
                const uint32_t voff = tv <= lim ? (in_blk + (uint32_t)tv) * hd.row_bytes : kOOB;
                tl.v[r] = Buf<VB>::stream(va, voff + vcol);
            }
        } else if constexpr (!PR) {
            const uint32_t in_blk = (uint32_t)(t0 & ((1 << hd.bs_shift) - 1));
            const uint32_t krow = j16 <= lim ? (in_blk + (uint32_t)j16) * hd.row_bytes : kOOB;
#pragma unroll
            for (int i = 0; i < KL; i++) tl.k[i] = Buf<16>::stream(ka, krow + kcol[i]);
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int tv = 4 * g4 + r;
                const uint32_t voff = tv <= lim ? (in_blk + (uint32_t)tv) * hd.row_bytes : kOOB;
                tl.v[r] = Buf<VB>::stream(va, voff + vcol);
            }
        } else {
            // Each access is issued against both blocks' descriptors; the one
            // not holding the row gets an out-of-range offset and reads 0.
            const rsrc_t kb = make_rsrc(hd.kbase + (size_t)pb * hd.blk_bytes, hd.rec_bytes);
            const rsrc_t vb = make_rsrc(hd.vbase + (size_t)pb * hd.blk_bytes, hd.rec_bytes);
            const bool live_k = j16 <= lim;
            const uint32_t ko = (uint32_t)(j16 & 7) * hd.row_bytes;
            const uint32_t koa = live_k && j16 < 8 ? ko : kOOB;
            const uint32_t kob = live_k && j16 >= 8 ? ko : kOOB;
#pragma unroll
            for (int i = 0; i < KL; i++)
                tl.k[i] = Buf<16>::stream(ka, koa + kcol[i]) | Buf<16>::stream(kb, kob + kcol[i]);
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int tv = 4 * g4 + r;
                const uint32_t vo = (uint32_t)(tv & 7) * hd.row_bytes;
                const uint32_t voa = tv <= lim && tv < 8 ? vo : kOOB;
                const uint32_t vob = tv <= lim && tv >= 8 ? vo : kOOB;
                tl.v[r] = Buf<VB>::stream(va, voa + vcol) | Buf<VB>::stream(vb, vob + vcol);
            }
        }
    }

    // Consumes one tile: scores, online softmax update, PV accumulate.  lim
    // as for issue(); rows past it get no weight.  CAUSAL: the B columns are
    // query tokens as well as heads, and column lane%16 also drops the rows
    // past clim (its own limit within the tile); a column can then have
    // seen no token yet, which the finite starting max of reset() covers.
    // MASK = false: the caller knows that every column it keeps sees every
    // row of the tile, so no limit is applied (the same result, fewer
    // vector instructions).
    // KLDS: kslot holds the tile's K rows (the loads complete).
    template <bool CAUSAL = false, bool MASK = true>
    __device__ inline void consume(Acc& a, const v8 (&qb)[KS], float scale_log2, int lim,
                                   const Tile& cur, int clim = 0,
                                   const lds_t* kslot = nullptr) const {
        u32x4 kf[KL];
        if constexpr (KLDS) {
#pragma unroll
            for (int i = 0; i < KL; i++) kf[i] = lds_read16(kslot + krd[i]);
        } else {
#pragma unroll
            for (int i = 0; i < KL; i++) kf[i] = cur.k[i];
        }
        const f32x4 sc = scores(qb, kf);
        v4 p_hi, p_lo;
        weights<CAUSAL, MASK>(a, sc, scale_log2, lim, clim, p_hi, p_lo);
        vrow vr[4];
        value_rows(cur, vr);
#pragma unroll
        for (int n = 0; n < NT; n++) {
            const v4 b = v4{vr[0][n], vr[1][n], vr[2][n], vr[3][n]};
            a.o[n] = M::pv(p_hi, b, a.o[n]);
        }
        if constexpr (M::kSplitP) {
#pragma unroll
            for (int n = 0; n < NT; n++) {
                const v4 b = v4{vr[0][n], vr[1][n], vr[2][n], vr[3][n]};
                a.o[n] = M::pv(p_lo, b, a.o[n]);
            }
        }
    }

  private:
    // The tile's four value rows of this lane (rows 4*g4 .. 4*g4+3, columns
    // NT*j16 ..), widened to the matrix-core type.
    __device__ inline void value_rows(const Tile& cur, vrow (&vr)[4]) const {
#pragma unroll
        for (int r = 0; r < 4; r++) {
            if constexpr (kFp8) {
                const uint32_t* w = (const uint32_t*)&cur.v[r];
#pragma unroll
                for (int q = 0; q < NT / 4; q++) {
                    const v4 x = M::from_fp8x4(w[q]);
#pragma unroll
                    for (int e = 0; e < 4; e++) vr[r][4 * q + e] = x[e];
                }
            } else {
                vr[r] = __builtin_bit_cast(vrow, cur.v[r]);
            }
        }
    }

    // Scores of the tile's 16 rows (K in the operand layout) against the 16 B
    // columns.
    __device__ inline f32x4 scores(const v8 (&qb)[KS], const u32x4 (&k)[KL]) const {
        f32x4 sc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int i = 0; i < KL; i++) {
            if constexpr (kFp8) {
                const v4 a0 = M::from_fp8x4(k[i][0]);
                const v4 a1 = M::from_fp8x4(k[i][1]);
                const v4 a2 = M::from_fp8x4(k[i][2]);
                const v4 a3 = M::from_fp8x4(k[i][3]);
                const v8 k0 = v8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
                const v8 k1 = v8{a2[0], a2[1], a2[2], a2[3], a3[0], a3[1], a3[2], a3[3]};
                sc = M::qk(k0, qb[2 * i], sc);
                sc = M::qk(k1, qb[2 * i + 1], sc);
            } else {
                sc = M::qk(__builtin_bit_cast(v8, k[i]), qb[i], sc);
            }
        }
        return sc;
    }

    // Masking, online softmax update of (m, l, o), and the weights as the A
    // operand (bf16 hi + lo pair where the type needs it).
    template <bool CAUSAL, bool MASK>
    __device__ inline void weights(Acc& a, const f32x4& sc, float scale_log2, int lim, int clim,
                                   v4& p_hi, v4& p_lo) const {
        float z[4];
        const int rlim = CAUSAL ? (clim < lim ? clim : lim) : lim;
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const float x = sc[r] * scale_log2;
            z[r] = (!MASK || 4 * g4 + r <= rlim) ? x : -INFINITY;
        }

        // ---- online softmax: tile max over the 16 tokens of each head ----
        // exp2 is the bare v_exp_f32 (results under 2^-126 flush to zero, a
        // weight far below what the sum can register); alpha is 0 at first.
        float mx = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
        mx = strided_max<16>(mx);
        const float m_new = mx > a.m + kTau ? mx : a.m;
        if (__any(m_new != a.m)) {
            const float alpha = m_new == a.m ? 1.0f : __builtin_amdgcn_exp2f(a.m - m_new);
            a.l *= alpha;
            // accumulator rows are heads 4*g4 + r; their alpha lives in lane 4*g4 + r
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const float ar = __shfl(alpha, 4 * g4 + r, 64);
#pragma unroll
                for (int n = 0; n < NT; n++) a.o[n][r] *= ar;
            }
            a.m = m_new;
        }
        float pz[4];
#pragma unroll
        for (int r = 0; r < 4; r++) pz[r] = __builtin_amdgcn_exp2f(z[r] - a.m);
        a.l += (pz[0] + pz[1]) + (pz[2] + pz[3]);

        // ---- weights as the A operand ----
#pragma unroll
        for (int r = 0; r < 4; r++) {
            p_hi[r] = (T)pz[r];
            if constexpr (M::kSplitP) p_lo[r] = (T)(pz[r] - (float)p_hi[r]);
        }
    }

  public:
    // Epilogue.  Lane (g4, j16) holds accumulator rows head = 4*g4 + r and
    // columns NT*j16 + n.  For every head < G, `out_row(head)` (when final)
    // receives the normalised row in the query type; otherwise `m_at(head)`,
    // `l_at(head)` and `o_at(head)` receive the partials (reference max in
    // natural-log units, sum, unnormalised output times v_scale).
    template <class OutRow, class MAt, class LAt, class OAt>
    __device__ inline void finish(const Acc& a, int G, bool final_out, float v_scale,
                                  OutRow out_row, MAt m_at, LAt l_at, OAt o_at) const {
        finish_each(a, G, [&](int) { return final_out; }, v_scale, out_row, m_at, l_at, o_at);
    }

    // As finish(), with the choice between the output row and the partials
    // made per column: final_of(head).  COMPACT: the partials take half the
    // bytes (the format of compact_entry); o_at(head) then points to D f16
    // values.
    template <bool COMPACT = false, class Final, class OutRow, class MAt, class LAt, class OAt>
    __device__ inline void finish_each(const Acc& a, int G, Final final_of, float v_scale,
                                       OutRow out_row, MAt m_at, LAt l_at, OAt o_at) const {
        const float l_tot = strided_sum<16>(a.l);     // head j16, over all tokens
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int head = 4 * g4 + r;
            const float lh = __shfl(l_tot, head, 64);
            const float mh = __shfl(a.m, head, 64);
            if (head >= G) continue;
            if (final_of(head)) {
                const float inv = lh > 0.0f ? v_scale / lh : 0.0f;   // no token seen: zeros
                vrow o;
#pragma unroll
                for (int n = 0; n < NT; n++) o[n] = (T)(a.o[n][r] * inv);
                *(vrow*)(out_row(head) + NT * j16) = o;
            } else if constexpr (COMPACT) {
                // the mean o / l of the row's 16 lanes (zeros where l = 0),
                // scaled by a power of two to the top octave below 2^15
                const float inv = lh > 0.0f ? v_scale / lh : 0.0f;
                float x[NT], am = 0.0f;
#pragma unroll
                for (int n = 0; n < NT; n++) {
                    x[n] = a.o[n][r] * inv;
                    am = fmaxf(am, fabsf(x[n]));
                }
                am = group_max<16>(am);
                const int e = compact_exponent(am);
                typedef _Float16 hrow __attribute__((ext_vector_type(NT)));
                hrow h;
#pragma unroll
                for (int n = 0; n < NT; n++) h[n] = (_Float16)__builtin_ldexpf(x[n], 15 - e);
                *(hrow*)(o_at(head) + NT * j16) = h;
                if (j16 == 0) {
                    *m_at(head) = mh * kLn2;
                    *l_at(head) = compact_l(lh, e);
                }
            } else {
                if (j16 == 0) {
                    *m_at(head) = mh * kLn2;
                    *l_at(head) = lh;
                }
                float* o = o_at(head) + NT * j16;
#pragma unroll
                for (int n = 0; n < NT; n++) o[n] = a.o[n][r] * v_scale;
            }
        }
    }
};

}  // namespace mfma
}  // namespace pkv
