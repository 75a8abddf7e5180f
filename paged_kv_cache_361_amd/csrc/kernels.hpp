// kernels.hpp - internal launch interface between the C ABI (api.hip) and the
// kernel translation units.  Not installed; the public contract is
// include/pagedkv.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

enum DType : int { kF32 = 0, kF16 = 1, kBF16 = 2, kFP8 = 3 };

struct WriteParams {
    const void* key;
    const void* value;
    void* k_cache;
    void* v_cache;
    const int64_t* slot_mapping;
    int64_t num_slots;     // num_blocks * block_size
    int T, Hkv, D;
    int src_bytes;         // bytes per source element
    float k_scale, v_scale;
};

struct DecodeParams {
    void* out;
    const void* q;
    const void* k;
    const void* v;
    const int32_t* tables;
    const int32_t* lens;
    float* ws_m;           // split-K partials (nullptr in one-pass mode)
    float* ws_l;
    float* ws_o;
    int32_t* ws_hdr;       // balanced mode: header of the workspace
    int32_t* ws_pre;       // balanced mode: tile prefix of the sequences [S + 1], then
                           // per stream (s * Hkv + h) its first chunk (bit 31: the
                           // chunk slot of its piece there) and its last chunk
    int nW;                // balanced mode: wavefronts of the persistent grid
    uint32_t epoch;        // balanced mode: this call's number (never repeats soon)
    const int32_t* q_start;  // multi-query: [S + 1] first query token of each sequence
    int max_groups;        // multi-query: wavefronts per (sequence, KV head) in the grid
    int col_blocks;        // multi-query: groups of 16 / G query tokens per wavefront
    int32_t* ws_len;       // multi-query split: tokens seen by each query token, for the reduce
    int len_rows;          // multi-query split: entries of ws_len (num_seqs * max_query_len)
    const int32_t* seq_bs; // mixed block sizes: tokens per block of each sequence [S]
    int page_shift;        // mixed block sizes: log2 of the pool's page (bs is the page)
    int S, Hq, Hkv, D, G, bs, NB, max_blocks;
    int len_cap;           // min(max_seq_len, max_blocks * bs)
    int P;                 // partition size, 0 = one pass
    int P_max;             // partitions per sequence covered by the grid
    float scale_log2;      // scale * k_scale * log2(e): scores in base-2 units
    float v_scale;
};

struct ReduceParams {
    void* out;
    const float* ws_m;
    const float* ws_l;
    const float* ws_o;
    const int32_t* ws_hdr; // balanced mode: header written by the decode call
    const int32_t* ws_pre; // balanced mode: tile prefix [S + 1] and stream chunk ranges
    const int32_t* lens;
    int S, Hq, Hkv, D, P, P_max, len_cap;
    int G, g_shift;        // balanced mode: Hq / Hkv, and its log2 (-1: not a power of 2)
    // balanced multi-query: rows are (query token, head), S counts query
    // tokens; the sequences' query_start [S_seq + 1] maps a token to its
    // sequence (nullptr: decode rows)
    const int32_t* q_start;
    int S_seq;
};

// ---- balanced split-K ------------------------------------------------------
//
// The T tiles of a batch (16 tokens of one (sequence, KV head) stream each,
// streams laid end to end) are cut into chunks by a guided schedule that
// depends only on T, the grid size nW and a floor F: nW chunks of C1 tiles
// (80% of an even share A = T / nW), then nW chunks of C2 = max(A / 7, F),
// then chunks of C3 = max(A / 16, F) up to T.  The decode sets F to two
// rounds of its tile ring, so that a chunk's index and table window, which
// arrive one after the other, are at hand before its first round is due.
// (Sizes measured best on MI355X for ragged batches on a grid of one wave
// per SIMD: neighbouring divisors were 1-15 us slower per call; on short fp8
// runs, floors of 4 and 12 tiles were 16 and 6 us slower than 20, and 30 or
// 40 slower again.)  Chunk c starts at tile
// chunk_begin(c), moved by the decode to a nearby stream end where one is
// close; the decode grid takes chunks 0..nW-1 statically and the rest from
// a counter, and records for every stream its first and last chunk, which
// is how the reduce finds a stream's entries.
//
// Workspace: a 256-byte header, the exclusive tile prefix of the sequences
// (S + 1 words) from byte 256 followed by two words per (sequence, KV head)
// stream (its first chunk, with the slot of its piece there in bit 31, and
// its last chunk), then (m, l, o) entries, two per query head of the group
// per chunk.  Header words 0-9 describe the split for the reduce
// (written by each decode call).  Words 32-33 (their own 128-byte line) hold
// the chunk counter, a 64-bit word: high half the number of the call that
// owns it, low half kCountTag | count.  Nothing resets it between calls: a
// call's first requests find another call's number (or whatever the memory
// held) and raise the word to the call's own base by a 64-bit max (call
// numbers increase; a word above the call's range is replaced by an
// exchange); every later request of the call adds one.  A stale word
// passes for live only if it carries the call's own 32-bit number and the
// 8-bit tag.
constexpr int32_t kBalancedMagic = 0x504B5642;
constexpr uint32_t kCountTag = 0xA5000000u;
constexpr uint32_t kCountMask = 0x00FFFFFFu;
enum BalancedHeader : int {
    kHdrMagic = 0, kHdrNW = 1, kHdrHkv = 2, kHdrG = 3, kHdrT = 4, kHdrC1 = 5, kHdrC2 = 6,
    kHdrC3 = 7, kHdrChunks = 8, kHdrFloor = 9, kHdrCounter = 32
};
// Largest chunk floor a decode sets (two rounds of its deepest ring).
constexpr int kMaxChunkFloor = 64;
// Upper bound on the persistent grid of the balanced kernel (wavefronts).
constexpr int kBalancedMaxWaves = 2048;
// Upper bound on the batch size of the balanced kernel (the tile prefix of
// the sequences is held in LDS).
constexpr int kBalancedMaxSeqs = 8192;

struct Sched {
    int T, nW, C1, C2, C3, chunks;
    int e1, e2;            // first tiles of the second and third phases (capped at T)
};

__host__ __device__ inline Sched make_sched(int T, int nW, int floor) {
    Sched q;
    q.T = T;
    q.nW = nW;
    const int A = nW > 0 ? T / nW : 0;
    q.C1 = A * 4 / 5 > 1 ? A * 4 / 5 : 1;
    if (floor < 4) floor = 4;
    q.C2 = A / 7 > floor ? A / 7 : floor;
    q.C3 = A / 16 > floor ? A / 16 : floor;
    const int64_t e1 = (int64_t)nW * q.C1;
    const int64_t e2 = e1 + (int64_t)nW * q.C2;
    q.e1 = (int)(e1 < T ? e1 : T);
    q.e2 = (int)(e2 < T ? e2 : T);
    if (T <= 0) q.chunks = 0;
    else if (e1 >= T) q.chunks = (T + q.C1 - 1) / q.C1;
    else if (e2 >= T) q.chunks = nW + (int)((T - e1 + q.C2 - 1) / q.C2);
    else q.chunks = 2 * nW + (int)((T - e2 + q.C3 - 1) / q.C3);
    return q;
}

// First tile of chunk c (c <= chunks; chunk_begin(chunks) == T).
__host__ __device__ inline int chunk_begin(const Sched& q, int c) {
    int64_t b;
    if (c <= q.nW) b = (int64_t)c * q.C1;
    else if (c <= 2 * q.nW) b = (int64_t)q.nW * q.C1 + (int64_t)(c - q.nW) * q.C2;
    else b = (int64_t)q.nW * (q.C1 + q.C2) + (int64_t)(c - 2 * q.nW) * q.C3;
    return (int)(b < q.T ? b : q.T);
}

// Most chunks any batch can produce on a grid of nW waves (the workspace
// bound): phases one and two hold 2 nW chunks; C1 + C2 > 0.94 A - 2, so the
// third covers fewer than (0.06 A + 3) nW tiles in chunks of at least
// max(4, A/16) (make_sched raises a floor below 4 to 4), fewer than
// 2 nW + 1 chunks for every A.  The bound keeps room to spare.
__host__ __device__ inline int64_t max_chunks(int nW) { return 5 * (int64_t)nW + 8; }

// Launches a kernel whose only parameter is a parameter struct and returns
// that launch's own status.
template <typename Kernel, typename Params>
inline hipError_t launch_kernel(Kernel kernel, dim3 grid, dim3 block, hipStream_t st,
                                const Params& p) {
    void* args[] = {const_cast<Params*>(&p)};
    return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, args, 0, st);
}

// Launchers; the caller has checked the matching *_supported() first.  They
// return hipErrorInvalidValue for a combination without a kernel.
hipError_t launch_reshape_and_cache(int src, int cache, const WriteParams& p, hipStream_t st);

// copy_blocks: whole blocks, src pools' block pairs[2i] -> dst pools' block
// pairs[2i + 1] (the pools may be the same, or one of them pinned host memory).
struct CopyParams {
    void* dk;
    void* dv;
    const void* sk;
    const void* sv;
    const int32_t* pairs;
    int n;                 // pairs
    int src_blocks, dst_blocks;
    uint32_t block_bytes;  // bytes of one block of one pool (a multiple of 16)
};
hipError_t launch_copy_blocks(const CopyParams& p, hipStream_t st);
bool decode_valu_supported(int qdt, int cdt, int D, int G);
hipError_t launch_decode_valu(int qdt, int cdt, const DecodeParams& p, hipStream_t st);
bool decode_mfma_supported(int qdt, int cdt, int D, int G);
hipError_t launch_decode_mfma(int qdt, int cdt, const DecodeParams& p, hipStream_t st);
// Mixed block sizes per sequence over a pool of pages (p.bs tokens each).
hipError_t launch_decode_mixed(int qdt, int cdt, const DecodeParams& p, hipStream_t st);
// Balanced mode (matrix-core kernel): resident wavefronts per CU of the
// kernel that would serve these types and shapes (0 if unknown), and launch.
int decode_balanced_waves_per_cu(int qdt, int cdt, int D, int bs, int S);
hipError_t launch_decode_balanced(int qdt, int cdt, const DecodeParams& p, hipStream_t st);
hipError_t launch_multi_query(int qdt, int cdt, const DecodeParams& p, hipStream_t st);
// Long query runs without a split, K/V staged in LDS (prefill.hip): query
// tokens per workgroup, the type combinations served, and the launch (one
// workgroup per (sequence, KV head, max_groups group)).
int prefill_tokens_per_group(int G);
bool prefill_supported(int qdt, int cdt, int D, int G);
hipError_t launch_prefill(int qdt, int cdt, const DecodeParams& p, hipStream_t st);
hipError_t launch_reduce(int out_dt, const ReduceParams& p, hipStream_t st);
hipError_t launch_reduce_balanced(int out_dt, const ReduceParams& p, hipStream_t st);

}  // namespace pkv
