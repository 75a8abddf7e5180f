// decode_mfma.hip - paged decode attention on the CDNA4 matrix cores.
//
// Same contract as the vector-ALU kernel (single query per sequence against
// its block-table-indirect K/V with an online softmax, "vLLM 推理引擎源码级拆解"
// §2.3), for f16/bf16 queries over f16/bf16/E4M3 caches.  A wavefront owns one
// unit = (sequence, KV head, partition) and serves the G <= 16 query heads of
// the GQA group with two matrix products per tile of 16 tokens:
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
// Memory side: per 16-token tile a wavefront issues D/32 16-byte K loads and 4
// V loads per lane, each instruction covering whole 64-byte (K) or 256-byte
// (V) row segments; the next tile's loads are issued before the current
// tile's arithmetic (one tile of prefetch per wavefront, 8 KiB for bf16
// D=128).  Block-table entries come in a 64-entry window held one per lane
// and are broadcast with readlane, so no dependent scalar load sits in front
// of every block.  Only the block base is wavefront-uniform (64-bit, scalar);
// per-lane offsets are 32-bit.
//
// E4M3 caches are widened to the query's 16-bit type with the gfx950 packed
// conversion (exact: every E4M3 value is a bf16 and an f16 value); the K and
// V scales are folded into the score scale and the output scale.
//
// With a bf16 query the softmax weights are fed as a bf16 pair hi + lo
// (hi = bf16(p), lo = bf16(p - hi)), i.e. ~16 significant bits, so the only
// 8-bit rounding left in the kernel is the stored output itself.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace pkv {
namespace {

constexpr int kWaves = 4;

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

template <class Q, class C, int D>
__global__ __launch_bounds__(64 * kWaves) void decode_mfma_kernel(DecodeParams p) {
    typedef Mfma<Q> M;
    typedef typename M::T T;
    typedef typename M::v8 v8;
    typedef typename M::v4 v4;
    constexpr bool kFp8 = std::is_same<C, FP8>::value;
    constexpr int EB = C::kBytes;         // cache bytes per element
    constexpr int KS = D / 32;            // QK contraction steps
    constexpr int NT = D / 16;            // PV column tiles = columns per lane
    constexpr int KL = kFp8 ? D / 64 : KS; // 16-byte K loads per lane per tile
    typedef T vrow __attribute__((ext_vector_type(NT)));           // NT values
    typedef uint8_t vrow8 __attribute__((ext_vector_type(NT)));     // NT codes
    typedef typename std::conditional<kFp8, vrow8, vrow>::type vraw;

    const int lane = threadIdx.x & 63;
    const int g4 = lane >> 4;             // lane group 0..3
    const int j16 = lane & 15;
    const int unit = blockIdx.x * kWaves + (threadIdx.x >> 6);
    const int h = unit % p.Hkv;
    const int rest = unit / p.Hkv;
    const int part = rest % p.P_max;
    const int s = rest / p.P_max;
    if (s >= p.S) return;

    const int G = p.G;
    int L = p.lens[s];
    L = L < p.len_cap ? L : p.len_cap;
    int t_begin = 0, t_end = L;
    bool final_out = true;
    if (p.P > 0) {
        const int nparts = L > 0 ? (L + p.P - 1) / p.P : 0;
        t_begin = part * p.P;
        t_end = min(L, t_begin + p.P);
        final_out = nparts <= 1;
    }
    T* out = (T*)p.out + ((size_t)s * p.Hq + (size_t)h * G) * D;
    if (L <= 0) {
        if (part == 0) {
            for (int i = lane; i < G * D; i += 64) out[i] = (T)0.0f;
        }
        return;
    }
    if (t_begin >= t_end) return;

    // --- query heads as the B operand of the score product ----------------
    v8 qb[KS];
    {
        const T* qrow = (const T*)p.q + ((size_t)s * p.Hq + (size_t)h * G + j16) * D;
#pragma unroll
        for (int kk = 0; kk < KS; kk++) {
            const int d0 = kFp8 ? (kk >> 1) * 64 + 16 * g4 + (kk & 1) * 8 : 32 * kk + 8 * g4;
            if (j16 < G) qb[kk] = *(const v8*)(qrow + d0);
            else qb[kk] = v8{};
        }
    }

    // --- addressing ---------------------------------------------------------
    const uint32_t row_bytes = (uint32_t)(p.Hkv * D * EB);   // bytes between slots
    const size_t blk_bytes = (size_t)p.bs * row_bytes;
    const char* kbase = (const char*)p.k + (size_t)h * D * EB;
    const char* vbase = (const char*)p.v + (size_t)h * D * EB;
    const int32_t* table = p.tables + (size_t)s * p.max_blocks;
    const uint32_t nb_last = (uint32_t)p.NB - 1u;
    const int bs = p.bs;
    const int bs_shift = bs == 8 ? 3 : (bs == 16 ? 4 : 5);
    const int nblk = (t_end + bs - 1) >> bs_shift;            // table entries used
    // Lane-constant parts of the offsets inside a slot row.
    uint32_t kcol[KL];
#pragma unroll
    for (int i = 0; i < KL; i++)
        kcol[i] = kFp8 ? (uint32_t)(64 * i + 16 * g4) : (uint32_t)((32 * i + 8 * g4) * EB);
    const uint32_t vcol = (uint32_t)(NT * j16 * EB);

    int win_base = t_begin >> bs_shift;
    int win = 0;
    if (win_base + lane < nblk) win = table[win_base + lane];

    // Loads of one tile into registers: K slices and V rows of this lane.
    struct Tile {
        u32x4 k[KL];
        vraw v[4];
    };
    auto load_tile = [&](int t0, Tile& tl) {
        const int blk = t0 >> bs_shift;
        if (blk + 1 - win_base >= 64) {               // slide the table window
            win_base = blk;
            win = (win_base + lane < nblk) ? table[win_base + lane] : 0;
        }
        const int lim = t_end - 1 - t0;               // last live token in tile
        uint32_t pa = (uint32_t)__builtin_amdgcn_readlane(win, blk - win_base);
        pa = pa < nb_last ? pa : nb_last;
        uint32_t pb = pa;
        if (bs == 8 && lim >= 8) {
            pb = (uint32_t)__builtin_amdgcn_readlane(win, blk + 1 - win_base);
            pb = pb < nb_last ? pb : nb_last;
        }
        const uint32_t in_blk = (uint32_t)(t0 & (bs - 1));
        const size_t base_a = (size_t)pa * blk_bytes;
        const size_t base_b = (size_t)pb * blk_bytes;
        // K row of token j16 (clamped to the last live token).
        {
            const int tk = j16 < lim ? j16 : lim;
            const bool in_b = bs == 8 && tk >= 8;
            const size_t base = in_b ? base_b : base_a;
            const uint32_t row = in_b ? (uint32_t)(tk - 8) : in_blk + (uint32_t)tk;
            const char* kp = kbase + base + (size_t)(row * row_bytes);
#pragma unroll
            for (int i = 0; i < KL; i++) tl.k[i] = *(const u32x4*)(kp + kcol[i]);
        }
        // V rows of tokens 4*g4 + r.
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int tv0 = 4 * g4 + r;
            const int tv = tv0 < lim ? tv0 : lim;
            const bool in_b = bs == 8 && tv >= 8;
            const size_t base = in_b ? base_b : base_a;
            const uint32_t row = in_b ? (uint32_t)(tv - 8) : in_blk + (uint32_t)tv;
            tl.v[r] = *(const vraw*)(vbase + base + (size_t)(row * row_bytes) + vcol);
        }
    };

    float m_run = -INFINITY;     // running max (base-2 units) of head j16
    float l_run = 0.0f;          // this lane's share of the running sum
    f32x4 acc[NT];
#pragma unroll
    for (int n = 0; n < NT; n++) acc[n] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    Tile cur, nxt;
    load_tile(t_begin, cur);
    for (int t0 = t_begin; t0 < t_end; t0 += 16) {
        if (t0 + 16 < t_end) load_tile(t0 + 16, nxt);

        // ---- scores ----
        f32x4 sc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int i = 0; i < KL; i++) {
            if constexpr (kFp8) {
                const v4 a0 = M::from_fp8x4(cur.k[i][0]);
                const v4 a1 = M::from_fp8x4(cur.k[i][1]);
                const v4 a2 = M::from_fp8x4(cur.k[i][2]);
                const v4 a3 = M::from_fp8x4(cur.k[i][3]);
                const v8 k0 = v8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
                const v8 k1 = v8{a2[0], a2[1], a2[2], a2[3], a3[0], a3[1], a3[2], a3[3]};
                sc = M::qk(k0, qb[2 * i], sc);
                sc = M::qk(k1, qb[2 * i + 1], sc);
            } else {
                sc = M::qk(__builtin_bit_cast(v8, cur.k[i]), qb[i], sc);
            }
        }
        const int lim = t_end - 1 - t0;
        float z[4];
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const float x = sc[r] * p.scale_log2;
            z[r] = (4 * g4 + r <= lim) ? x : -INFINITY;
        }

        // ---- online softmax: tile max over the 16 tokens of each head ----
        float mx = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
        mx = strided_max<16>(mx);
        const float m_new = fmaxf(m_run, mx);
        if (__any(m_new > m_run)) {
            const float alpha = exp2f(m_run - m_new);   // 0 on the first tile
            l_run *= alpha;
            // accumulator rows are heads 4*g4 + r; their alpha lives in lane 4*g4 + r
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const float ar = __shfl(alpha, 4 * g4 + r, 64);
#pragma unroll
                for (int n = 0; n < NT; n++) acc[n][r] *= ar;
            }
            m_run = m_new;
        }
        float pz[4];
#pragma unroll
        for (int r = 0; r < 4; r++) pz[r] = exp2f(z[r] - m_run);
        l_run += (pz[0] + pz[1]) + (pz[2] + pz[3]);

        // ---- weights as the A operand, value rows as the B operand ----
        v4 p_hi, p_lo;
#pragma unroll
        for (int r = 0; r < 4; r++) {
            p_hi[r] = (T)pz[r];
            if constexpr (M::kSplitP) p_lo[r] = (T)(pz[r] - (float)p_hi[r]);
        }
        vrow vr[4];
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
                vr[r] = cur.v[r];
            }
        }
#pragma unroll
        for (int n = 0; n < NT; n++) {
            const v4 b = v4{vr[0][n], vr[1][n], vr[2][n], vr[3][n]};
            acc[n] = M::pv(p_hi, b, acc[n]);
        }
        if constexpr (M::kSplitP) {
#pragma unroll
            for (int n = 0; n < NT; n++) {
                const v4 b = v4{vr[0][n], vr[1][n], vr[2][n], vr[3][n]};
                acc[n] = M::pv(p_lo, b, acc[n]);
            }
        }
        cur = nxt;
    }

    // ---- epilogue: lane (g4, j16) holds rows 4*g4 + r, columns NT*j16 + n ----
    const float l_tot = strided_sum<16>(l_run);     // head j16, over all tokens
#pragma unroll
    for (int r = 0; r < 4; r++) {
        const int head = 4 * g4 + r;
        const float lh = __shfl(l_tot, head, 64);
        const float mh = __shfl(m_run, head, 64);
        if (head >= G) continue;
        if (final_out) {
            const float inv = p.v_scale / lh;
            vrow o;
#pragma unroll
            for (int n = 0; n < NT; n++) o[n] = (T)(acc[n][r] * inv);
            *(vrow*)(out + (size_t)head * D + NT * j16) = o;
        } else {
            const size_t idx = ((size_t)s * p.Hq + (size_t)h * G + head) * p.P_max + part;
            if (j16 == 0) {
                p.ws_m[idx] = mh * kLn2;
                p.ws_l[idx] = lh;
            }
            float* o = p.ws_o + idx * D + NT * j16;
#pragma unroll
            for (int n = 0; n < NT; n++) o[n] = acc[n][r] * p.v_scale;
        }
    }
}

template <class Q, class C>
hipError_t launch_d(const DecodeParams& p, hipStream_t st) {
    const long units = (long)p.S * p.P_max * p.Hkv;
    const dim3 grid((unsigned)((units + kWaves - 1) / kWaves)), block(64 * kWaves);
    if (p.D == 64) return launch_kernel(decode_mfma_kernel<Q, C, 64>, grid, block, st, p);
    if (p.D == 128) return launch_kernel(decode_mfma_kernel<Q, C, 128>, grid, block, st, p);
    return hipErrorInvalidValue;
}

}  // namespace

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
