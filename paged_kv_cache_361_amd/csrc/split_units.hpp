// split_units.hpp - the split-K work list shared by the per-unit kernels
// (decode_mfma.hip, multi_query.hip): with partition size P > 0, sequence s
// contributes max(1, ceil(L_s / P)) (sequence, partition) pairs, every
// full-length partition first and the last, ragged partition of each
// sequence after them, so short units fill the tail of a grid.
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace pkv {

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

// Maps the sp-th (sequence, partition) pair of the split-K work list.  The
// list holds first every partition that is not the last one of its sequence
// (all exactly P tokens), sequence-major, then the last partition of each
// sequence in sequence order.  Each lane owns 4 consecutive sequences of a
// 256-sequence chunk; a wavefront prefix sum of the per-lane counts of
// leading partitions locates a pair of the first kind.  Returns false when
// sp is past the end of the list.
__device__ inline bool find_unit(const DecodeParams& p, int sp, int* s_out, int* part_out) {
    const int lane = threadIdx.x & 63;
    int before = 0;                       // leading partitions in earlier chunks
    for (int c0 = 0; c0 < p.S; c0 += 256) {
        int n[4];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int s = c0 + 4 * lane + i;
            n[i] = s < p.S ? seq_parts(p, p.lens[s]) - 1 : 0;
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
    const int s = sp - before;            // last partition of sequence s
    if (s >= p.S) return false;
    *s_out = s;
    *part_out = seq_parts(p, p.lens[s]) - 1;
    return true;
}

}  // namespace pkv
