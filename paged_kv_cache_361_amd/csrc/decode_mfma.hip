// decode_mfma.hip - paged decode attention on the CDNA4 matrix cores.
//
// Same contract as the vector-ALU kernel (single query per sequence against
// its block-table-indirect K/V with an online softmax, "vLLM 推理引擎源码级拆解"
// §2.3), for f16/bf16 queries over f16/bf16/E4M3 caches.  A wavefront owns one
// unit = (sequence, partition, KV head) and serves the G <= 16 query heads of
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
// Memory side.  Every K/V access is a buffer load whose 128-bit descriptor
// holds the 64-bit base of one physical block (plus the head offset) in
// scalar registers, with 32-bit per-lane offsets inside the block.  Rows past
// the end of the unit get an offset beyond the descriptor's range: the
// hardware returns zeros without touching memory, so masked tokens cost no
// bandwidth and whatever the pool holds there (NaN poison included) never
// reaches the arithmetic.  Two tiles are in flight per wavefront: the loop is
// unrolled by hand into an A/B pair so that the loads of one tile are issued
// before the other tile is consumed and no register copy forces an early
// wait.  Block ids come from a 64-entry window of the block table held one
// entry per lane and broadcast with readlane.
//
// Split-K work list.  With partition_size P > 0, sequence s contributes
// max(1, ceil(L_s / P)) partitions.  The (sequence, partition) pairs are
// numbered sequence-major without gaps, so every wavefront of the grid that
// has work owns a full unit and the ragged lengths of a batch become units of
// at most P tokens; waves numbered past the total exit at once.  Each wave
// finds its pair from the lengths with a wavefront prefix sum.
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
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace pkv {
namespace {

constexpr int kWaves = 4;
constexpr float kTau = 8.0f;            // lazy-rescale threshold (base-2 units)
constexpr uint32_t kOOB = 0x80000000u;  // past any descriptor range: reads 0

typedef __amdgpu_buffer_rsrc_t rsrc_t;

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
};
template <>
struct Buf<8> {
    typedef u32x2 T;
    __device__ static inline T load(rsrc_t r, uint32_t off) {
        return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0));
    }
};
template <>
struct Buf<4> {
    typedef uint32_t T;
    __device__ static inline T load(rsrc_t r, uint32_t off) {
        return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
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

// Inclusive prefix sum over the 64 lanes of a wavefront.
__device__ inline int wave_incl_scan(int x) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    return x;
}

// Partitions of sequence s in split-K mode: max(1, ceil(L / P)) with L
// clamped to the grid's length bound; a sequence with no tokens keeps one
// unit, which writes its zero row.
__device__ inline int seq_parts(const DecodeParams& p, int L) {
    L = L < p.len_cap ? L : p.len_cap;
    return L > 0 ? (L + p.P - 1) / p.P : 1;
}

// The sp-th (sequence, partition) pair in sequence-major order.  Each lane
// owns 4 consecutive sequences of a 256-sequence chunk; a wavefront prefix sum
// of the per-lane partition counts locates the pair.  Returns false when sp
// is past the last pair.
__device__ inline bool find_unit(const DecodeParams& p, int sp, int* s_out, int* part_out) {
    const int lane = threadIdx.x & 63;
    int before = 0;                       // pairs in earlier chunks
    for (int c0 = 0; c0 < p.S; c0 += 256) {
        int n[4];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int s = c0 + 4 * lane + i;
            n[i] = s < p.S ? seq_parts(p, p.lens[s]) : 0;
        }
        const int mine = (n[0] + n[1]) + (n[2] + n[3]);
        const int incl = wave_incl_scan(mine);
        const int total = __shfl(incl, 63, 64);
        if (sp < before + total) {
            const uint64_t hit = __ballot(before + incl > sp);
            const int l = (int)__builtin_ctzll(hit);
            int k = sp - before - __shfl(incl - mine, l, 64);   // index within lane l
            int s = c0 + 4 * l;
#pragma unroll
            for (int i = 0; i < 3; i++) {
                const int ni = __shfl(n[i], l, 64);
                if (k >= ni) {
                    k -= ni;
                    s++;
                } else {
                    break;
                }
            }
            *s_out = s;
            *part_out = k;
            return true;
        }
        before += total;
    }
    return false;
}

// PAIR: block size 8, so a 16-token tile spans two blocks.
template <class Q, class C, int D, bool PAIR>
__global__ __launch_bounds__(64 * kWaves) void decode_mfma_kernel(DecodeParams p) {
    typedef Mfma<Q> M;
    typedef typename M::T T;
    typedef typename M::v8 v8;
    typedef typename M::v4 v4;
    constexpr bool kFp8 = std::is_same<C, FP8>::value;
    constexpr int EB = C::kBytes;          // cache bytes per element
    constexpr int KS = D / 32;             // QK contraction steps
    constexpr int NT = D / 16;             // PV column tiles = columns per lane
    constexpr int KL = kFp8 ? D / 64 : KS; // 16-byte K loads per lane per tile
    constexpr int VB = NT * EB;            // bytes of one V row slice per lane
    typedef T vrow __attribute__((ext_vector_type(NT)));   // NT values
    typedef typename Buf<VB>::T vraw;

    const int lane = threadIdx.x & 63;
    const int g4 = lane >> 4;              // lane group 0..3
    const int j16 = lane & 15;
    // Everything that selects the unit is wave-uniform; readfirstlane tells
    // the compiler so, which keeps block descriptors in scalar registers.
    const int unit = blockIdx.x * kWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = unit % p.Hkv;
    const int sp = unit / p.Hkv;
    int s = sp, part = 0;
    if (p.P > 0) {
        if (!find_unit(p, sp, &s, &part)) return;
        s = __builtin_amdgcn_readfirstlane(s);
        part = __builtin_amdgcn_readfirstlane(part);
    } else if (s >= p.S) {
        return;
    }

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
    const uint32_t head_off = (uint32_t)(h * D * EB);
    const uint32_t blk_bytes = (uint32_t)p.bs * row_bytes;
    const uint32_t rec_bytes = blk_bytes - head_off;          // descriptor range
    const char* kbase = (const char*)p.k + head_off;
    const char* vbase = (const char*)p.v + head_off;
    const int32_t* table = p.tables + (size_t)s * p.max_blocks;
    const uint32_t nb_last = (uint32_t)p.NB - 1u;
    const int bs = p.bs;
    const int bs_shift = bs == 8 ? 3 : (bs == 16 ? 4 : 5);
    const int nblk = (t_end + bs - 1) >> bs_shift;             // table entries used
    // Lane-constant parts of the offsets inside a slot row.
    uint32_t kcol[KL];
#pragma unroll
    for (int i = 0; i < KL; i++)
        kcol[i] = kFp8 ? (uint32_t)(64 * i + 16 * g4) : (uint32_t)((32 * i + 8 * g4) * EB);
    const uint32_t vcol = (uint32_t)(NT * j16 * EB);

    struct Tile {
        u32x4 k[KL];
        vraw v[4];
    };
    // Issues the loads of the tile starting at token t0 (no wait); the
    // block ids come from `win`, the table entries from block wb on.  Rows
    // at or past w_end, and every row of a tile past it, read as zeros.
    auto issue = [&](int t0, int w_end, int wb, int win, Tile& tl) {
        const int lim = w_end - 1 - t0;                 // last live row (<0: none)
        uint32_t pa = 0, pb = 0;
        if (lim >= 0) {
            const int blk = (t0 >> bs_shift) - wb;
            pa = (uint32_t)__builtin_amdgcn_readlane(win, blk);
            pa = pa < nb_last ? pa : nb_last;
            if (PAIR && lim >= 8) {
                pb = (uint32_t)__builtin_amdgcn_readlane(win, blk + 1);
                pb = pb < nb_last ? pb : nb_last;
            }
        }
        const rsrc_t ka = make_rsrc(kbase + (size_t)pa * blk_bytes, rec_bytes);
        const rsrc_t va = make_rsrc(vbase + (size_t)pa * blk_bytes, rec_bytes);
        if constexpr (!PAIR) {
            const uint32_t in_blk = (uint32_t)(t0 & (bs - 1));
            const uint32_t krow = j16 <= lim ? (in_blk + (uint32_t)j16) * row_bytes : kOOB;
#pragma unroll
            for (int i = 0; i < KL; i++) tl.k[i] = Buf<16>::load(ka, krow + kcol[i]);
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int tv = 4 * g4 + r;
                const uint32_t vrow_off = tv <= lim ? (in_blk + (uint32_t)tv) * row_bytes : kOOB;
                tl.v[r] = Buf<VB>::load(va, vrow_off + vcol);
            }
        } else {
            // Each access is issued against both blocks' descriptors; the one
            // not holding the row gets an out-of-range offset and reads 0.
            const rsrc_t kb = make_rsrc(kbase + (size_t)pb * blk_bytes, rec_bytes);
            const rsrc_t vb = make_rsrc(vbase + (size_t)pb * blk_bytes, rec_bytes);
            const bool live_k = j16 <= lim;
            const uint32_t ko = (uint32_t)(j16 & 7) * row_bytes;
            const uint32_t koa = live_k && j16 < 8 ? ko : kOOB;
            const uint32_t kob = live_k && j16 >= 8 ? ko : kOOB;
#pragma unroll
            for (int i = 0; i < KL; i++)
                tl.k[i] = Buf<16>::load(ka, koa + kcol[i]) | Buf<16>::load(kb, kob + kcol[i]);
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int tv = 4 * g4 + r;
                const uint32_t vo = (uint32_t)(tv & 7) * row_bytes;
                const uint32_t voa = tv <= lim && tv < 8 ? vo : kOOB;
                const uint32_t vob = tv <= lim && tv >= 8 ? vo : kOOB;
                tl.v[r] = Buf<VB>::load(va, voa + vcol) | Buf<VB>::load(vb, vob + vcol);
            }
        }
    };

    float m_run = -INFINITY;     // reference max (base-2 units) of head j16
    float l_run = 0.0f;          // this lane's share of the running sum
    f32x4 acc[NT];
#pragma unroll
    for (int n = 0; n < NT; n++) acc[n] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // Consumes one tile: scores, online softmax update, PV accumulate.
    auto consume = [&](int t0, const Tile& cur) {
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
        const float m_new = mx > m_run + kTau ? mx : m_run;
        if (__any(m_new != m_run)) {
            const float alpha = m_new == m_run ? 1.0f : exp2f(m_run - m_new);  // 0 at first
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
                vr[r] = __builtin_bit_cast(vrow, cur.v[r]);
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
    };

    // ---- two tiles in flight: A/B ping-pong, loads always issued ----------
    // The unit is walked in windows of 64 table entries (one per lane); a
    // split-K partition of at most 64 blocks is a single window.
    const int wtok = 64 << bs_shift;
    for (int w0 = t_begin; w0 < t_end; w0 += wtok) {
        const int w1 = min(t_end, w0 + wtok);
        const int wb = w0 >> bs_shift;
        const int win = (wb + lane < nblk) ? table[wb + lane] : 0;
        Tile ta, tb;
        issue(w0, w1, wb, win, ta);
        issue(w0 + 16, w1, wb, win, tb);
        for (int t0 = w0; t0 < w1; t0 += 32) {
            consume(t0, ta);
            issue(t0 + 32, w1, wb, win, ta);
            if (t0 + 16 < w1) consume(t0 + 16, tb);
            issue(t0 + 48, w1, wb, win, tb);
        }
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
    const bool pair = p.bs == 8;
    if (p.D == 64)
        return pair ? launch_kernel(decode_mfma_kernel<Q, C, 64, true>, grid, block, st, p)
                    : launch_kernel(decode_mfma_kernel<Q, C, 64, false>, grid, block, st, p);
    if (p.D == 128)
        return pair ? launch_kernel(decode_mfma_kernel<Q, C, 128, true>, grid, block, st, p)
                    : launch_kernel(decode_mfma_kernel<Q, C, 128, false>, grid, block, st, p);
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
