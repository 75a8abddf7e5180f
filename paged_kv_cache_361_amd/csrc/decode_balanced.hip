// decode_balanced.hip - paged decode attention with the work of a whole
// batch spread over a persistent grid of wavefronts by a guided dynamic
// schedule ("balanced" split-K, partition_size = PKV_PARTITION_BALANCED).
//
// What is computed is the same single-query attention through the block
// table as in "vLLM 推理引擎源码级拆解" §2.3; only the division of the work
// differs.  Every (sequence, KV head) pair is a stream of 16-token tiles;
// the streams are laid end to end (sequence-major, then KV head) and the
// resulting T tiles are cut into chunks by the guided schedule of
// kernels.hpp: nW chunks of the first size, nW of the second, then small
// ones.  The grid holds one wavefront per SIMD of the GPU (nW);
// wave w works on chunk w, then takes chunks in order from a counter in the
// workspace.  Waves of one GPU do not stream at one rate (on a loaded GPU
// some take nearly twice as long as others over the same tiles), so the
// smaller chunks that follow keep every wave busy until the batch is done.
// Adds to the one counter are serialised (about 12 ns each), so a wave asks
// for its next chunk only when a few rounds of its current one are left:
// requests from all waves at once would delay the last by tens of
// microseconds.
//
// A piece of a stream inside one chunk is a segment.  A segment that is a
// whole stream writes its output rows directly.  Any other segment is the
// first or the last of its chunk and writes its partials (reference max,
// sum, unnormalised output) to slot 0 (first) or 1 (last) of the chunk in the
// workspace; pkv_paged_attention_reduce merges, for each stream spread over
// chunks c0..c1, the entries of those chunks.
//
// One kernel per call.  Every workgroup computes the tile prefix of the
// sequences in LDS; workgroup 0 also writes it and the schedule into the
// workspace for the reduce.  The chunk counter needs no reset before the
// call (no memset, so the call can be captured in a graph): it carries the
// number of the call that owns it, and the call's first request takes it
// over (kernels.hpp).  The reduce that follows returns it to zero, which is
// what lets a replayed graph, whose call number never changes, take it over
// again.
//
// Pipeline.  The matrix-core tile of tile_mfma.hpp runs on a ring of DEPTH
// tile buffers.  Segments are cut into spans of at most 64 blocks (one
// block-table window, one entry per lane) and spans into rounds of DEPTH
// tiles (the last round of a span padded with dead tiles).  The producer
// issues round r + 1 while the consumer works through round r, slot by
// slot, across span, segment and chunk boundaries: the table window of the
// producer's next span, the query rows of a segment it enters and the index
// of the chunk after its current one (the counter's atomic add) are all
// requested one step ahead, and the lengths and tile prefix the walk needs
// are held in LDS, so moving on never drains the ring.
//
// K tiles in LDS.  Where the ring's K slots fit beside the prefix arrays
// (16-byte caches at head_dim 128: 96 KiB per workgroup, so up to about 8,000
// sequences, 5,400 with query starts or geometries), the K rows go from
// memory straight into a slot of LDS in row order and are read back in the
// operand layout (TileMath<..., KLDS>); V stays in registers.  A 16-token
// tile over two 8-token blocks does the same where each row-order load
// covers rows of one block (at most 8 rows a load).  The loads
// carry no register the compiler could wait on, so the consumer waits with
// an explicit count before reading slot j: every round issues all DEPTH
// tiles in ring order (dead tiles read nothing but still count), so once at
// most the loads of the DEPTH - 1 tiles issued after slot j's are in flight,
// slot j's are done.  Scheduling barriers keep whole tiles in ring order.
// On MI355X this took the 40-head MHA layer from 297.7 to 271.2 µs per call
// (decode + reduce) and the mixed-block-size batch from 253.5 to 251.8; the
// 8-head GQA layers read alike either way (246.7 against 245.3 µs, long
// contexts 430.3 against 433.9).
#include "split_units.hpp"
#include "tile_mfma.hpp"

namespace pkv {
namespace {

using namespace mfma;

constexpr int kWaves = 4;
// Tiles before the end of its chunk at which a wave asks for its next one.
// Stepping into the next chunk without a stall needs about three rounds
// (the index, then the table window of its first span), and a request's
// latency is about one round when requests are spread out; asking earlier
// only lengthens the work a wave still holds when the chunks run out (4 to
// 8 tiles measured alike on MI355X, 12 about 4 us slower per batch).
constexpr int kRequestAhead = 8;

// Atomic add on a buffer word, returning the old value; lanes whose offset
// is past the descriptor's range do nothing (and read 0).  Used with only
// lane 0 in range, so the wave adds once without a branch around the
// instruction (a branch around a memory instruction would cost the loop a
// full wait on every load in flight).
__device__ long long buffer_atomic_add_i64(long long v, rsrc_t r, int off, int soff, int aux)
    __asm("llvm.amdgcn.raw.ptr.buffer.atomic.add.i64");

// The chunk counter (kernels.hpp): whether a value read from it belongs to
// call `epoch`.
__device__ inline bool counter_live(uint64_t v, uint32_t epoch) {
    return (uint32_t)(v >> 32) == epoch && ((uint32_t)v & ~kCountMask) == kCountTag;
}

// A request found the counter not yet this call's.  Call numbers increase,
// so the call's range of values, (epoch << 32 | kCountTag) and up, lies
// above whatever an earlier call left: a 64-bit max installs the call's base
// whoever gets there first (and undoes any stale adds), then an add takes an
// index as usual.  A word above the call's range (memory never written by a
// call, another mode's data, or call numbers wrapping round) is replaced by
// an exchange that takes index 0.  At most three atomics and no retry loop,
// so no number of wavefronts arriving together can keep one waiting.  Two
// exchanges in one call can hand out some indices twice; a chunk computed
// twice writes the same values twice, and no index is ever skipped.
__device__ inline int counter_rebase(unsigned long long* ctr, uint32_t epoch) {
    int k = 0;
    if ((threadIdx.x & 63) == 0) {
        const unsigned long long base = ((unsigned long long)epoch << 32) | kCountTag;
        atomicMax(ctr, base);
        const unsigned long long old = atomicAdd(ctr, 1ull);
        if (counter_live(old, epoch)) k = (int)((uint32_t)old & kCountMask);
        else atomicExch(ctr, base | 1u);          // k = 0
    }
    return __builtin_amdgcn_readfirstlane(k);
}

// Tiles of a sequence of L tokens in tiles of 2^ts tokens (ts = 4: 16-token
// tiles; ts = 3: the 8-token tiles of 8-token blocks with mixed block sizes).
__device__ inline int seq_tiles(int L, int ts = 4) { return L > 0 ? (L + (1 << ts) - 1) >> ts : 0; }

// Mixed block sizes: a sequence's geometry, packed in one LDS word: log2 of
// its block size (low byte) and of its tile (next byte).  A block of 8
// tokens takes 8-token tiles (rows 8-15 of the 16-row matrix-core tile
// dead), so that every tile lies inside one block; 16- and 32-token blocks
// take 16-token tiles.  Uniform pools pass the pool's block size.
__device__ inline int geo_pack(int shift, int ts) { return shift | (ts << 8); }
__device__ inline int geo_shift(int g) { return g & 255; }
__device__ inline int geo_ts(int g) { return g >> 8; }
// The same in 3 bits (block shift 3..5, tile shift 3..4), kept in a span's
// key above the sequence and head (no extra scalar register per span).
__device__ inline int geo_code(int g) { return (geo_shift(g) - 3) | ((geo_ts(g) - 3) << 2); }
__device__ inline int code_shift(int c) { return (c & 3) + 3; }
__device__ inline int code_ts(int c) { return (c >> 2) + 3; }

// A copy of a loaded value made by an instruction the compiler cannot see
// through, so that it waits for that one load here.  Used on rare paths
// whose loaded registers merge into the main loop: without it the compiler
// would treat the register as possibly in flight on the common path too and
// wait there for every load issued.
__device__ inline int settled(int x) {
    int y;
    asm volatile("v_mov_b32 %0, %1" : "=v"(y) : "v"(x));
    return y;
}

// Bytes of the kernel's LDS arrays: the tile prefix and the lengths, plus
// query_start (MULTI) or the geometries (MIXED); LDS-staged K slots start at
// the next 256-byte boundary.
__host__ __device__ constexpr size_t lds_bytes(int S, bool wide) {
    return (size_t)((wide ? 3 : 2) * S + (wide ? 2 : 1)) * sizeof(int);
}
__host__ __device__ constexpr size_t ring_offset(int S, bool wide) {
    return (lds_bytes(S, wide) + 255) & ~(size_t)255;
}

// ---- tile prefix ----------------------------------------------------------

// Every workgroup computes the batch's tile prefix in LDS from the lengths:
// len[s] = clamped length of sequence s, pre[s] = tiles of the streams of
// all sequences before s (pre[S] = T).  MIXED: geo[s] = the sequence's
// geometry (its block size from p.seq_bs, as decode_mixed_kernel reads it),
// and its length is also clamped to what its table can hold.
template <bool MIXED>
__device__ inline void wg_prefix(const DecodeParams& p, int* pre, int* len, int* geo) {
    __shared__ int wave_sum[kWaves];
    constexpr int NT = 64 * kWaves;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;
    // lengths into LDS with coalesced loads, then a scan over contiguous
    // ranges of `per` sequences per thread
#pragma unroll 4
    for (int s = tid; s < p.S; s += NT) {
        int L = min(p.lens[s], p.len_cap);
        if constexpr (MIXED) {
            const int bs = p.seq_bs[s];
            const int shift = bs >= 32 ? 5 : max(bs >= 16 ? 4 : 3, p.page_shift);
            geo[s] = geo_pack(shift, shift == 3 ? 3 : 4);
            L = min(L, p.max_blocks << shift);
        }
        len[s] = L;
    }
    __syncthreads();
    const int per = (p.S + NT - 1) / NT;
    const int s0 = tid * per;
    int n = 0;
    for (int i = 0; i < per; i++) {
        const int s = s0 + i;
        if (s < p.S) n += seq_tiles(len[s], MIXED ? geo_ts(geo[s]) : 4) * p.Hkv;
    }
    const int incl = wave_incl_scan(n);
    if (lane == 63) wave_sum[wv] = incl;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int k = 0; k < kWaves; k++) {
        before += k < wv ? wave_sum[k] : 0;
        total += wave_sum[k];
    }
    int run = before + incl - n;
    for (int i = 0; i < per; i++) {
        const int s = s0 + i;
        if (s < p.S) {
            pre[s] = run;
            run += seq_tiles(len[s], MIXED ? geo_ts(geo[s]) : 4) * p.Hkv;
        }
    }
    if (tid == 0) pre[p.S] = total;
    __syncthreads();
}

// First tile of chunk c: the schedule's chunk_begin, moved to the nearer
// end of the stream it falls in when that end lies within an eighth of the
// smaller of the two chunks it separates (a quarter between the later,
// dynamically taken chunks).  A cut inside a stream costs the stream two
// partial entries (written here, read by the reduce).  Moving a cut changes
// two chunks' sizes; the first nW chunks are each wave's fixed share, which
// bears little of that (MI355X: a quarter there cost the long-context batch
// 6% and the MHA batch 2%, an eighth nothing), while the later ones are
// taken as waves free up.  Verification (MULTI) moves every cut within a
// quarter: its partial entries hold 16 rows instead of G, four times the
// bytes per cut stream.  Chunks stay non-empty (each keeps at least half
// its tiles), chunk 0 starts at 0 and the last ends at T; the reduce reads
// each stream's chunks from what the decode records, so it needs no copy of
// this rule.
template <bool MULTI>
__device__ inline int chunk_start(const Sched& q, int c, const int* pre, const int* len,
                                   const int* geo, int S) {
    const int b = chunk_begin(q, c);
    if (c <= 0 || c >= q.chunks) return b;
    const int d = min(b - chunk_begin(q, c - 1), chunk_begin(q, c + 1) - b) /
                  (c <= q.nW && !MULTI ? 8 : 4);
    if (d <= 0) return b;
    int lo = 0, hi = S;                    // pre[lo] <= b < pre[lo + 1]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (__builtin_amdgcn_readfirstlane(pre[mid]) <= b) lo = mid;
        else hi = mid;
    }
    const int ts = geo ? geo_ts(__builtin_amdgcn_readfirstlane(geo[lo])) : 4;
    const int nt = seq_tiles(__builtin_amdgcn_readfirstlane(len[lo]), ts);
    const int r = (b - __builtin_amdgcn_readfirstlane(pre[lo])) % nt;
    if (r <= d) return b - r;
    if (nt - r <= d) return b + nt - r;
    return b;
}

// ---- decode ----------------------------------------------------------------

// Span flags.
enum : int { kFirst = 1, kLast = 2, kComplete = 4, kSlot1 = 8, kStart = 16, kEnd = 32 };

// A span: tiles [t0, t1) of stream (s, h) (packed in `key`), within one table
// window starting at block wb, inside chunk `chunk`.  Wave-uniform; kept
// small because three of them live in scalar registers.
struct Span {
    int key;           // geometry code (mixed block sizes) << 25 | s << 12 | h
    int L, t0, t1, wb, chunk;
    int flags;         // kFirst: first span of its segment; kLast: last;
                       // kComplete: the segment is the whole stream;
                       // kSlot1: not the first segment of its chunk;
                       // (last span) kStart: the segment starts the stream,
                       // kEnd: it ends it
    template <bool MIXED>
    __device__ int seq() const { return MIXED ? (key >> 12) & 0x1FFF : key >> 12; }
    __device__ int s() const { return (key >> 12) & 0x1FFF; }
    __device__ int h() const { return key & 4095; }
    __device__ int code() const { return key >> 25; }
};

// Wave-uniform walk over one chunk, span by span.  pre and len are the LDS
// copies of the tile prefix and of the clamped lengths; geo those of the
// sequences' geometries (nullptr: every sequence has geometry `g0`).
struct Walk {
    int s, h, tile;    // next tile: stream (s, h), tile index
    int L;             // clamped length of sequence s
    int g;             // its geometry (geo_pack)
    int rem;           // tiles of the chunk not yet walked
    int chunk;
    int wf;            // 1: the current segment continues in the next span;
                       // 2: it started at tile 0; 4: a segment already ended
                       // in this chunk

    __device__ inline void start(const int* pre, const int* len, const int* geo, int g0, int S,
                                 int c, int x0, int x1) {
        // the sequence whose streams hold tile x0: pre[s] <= x0 < pre[s + 1]
        int lo = 0, hi = S;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (__builtin_amdgcn_readfirstlane(pre[mid]) <= x0) lo = mid;
            else hi = mid;
        }
        s = lo;
        L = __builtin_amdgcn_readfirstlane(len[s]);
        g = geo ? __builtin_amdgcn_readfirstlane(geo[s]) : g0;
        const int nt = seq_tiles(L, geo ? geo_ts(g) : 4);
        const int off = x0 - __builtin_amdgcn_readfirstlane(pre[s]);
        h = off / nt;
        tile = off % nt;
        rem = x1 - x0;
        chunk = c;
        wf = 0;
    }

    __device__ inline bool next(const int* len, const int* geo, int S, int Hkv, int bs_shift,
                                Span& o) {
        if (rem <= 0) return false;
        int nt = seq_tiles(L, geo ? geo_ts(g) : 4);
        while (tile >= nt) {               // stream exhausted: move on
            tile = 0;
            wf &= ~1;
            if (++h == Hkv) {
                h = 0;
                do {
                    if (++s >= S) return false;    // not reached while rem > 0
                    L = __builtin_amdgcn_readfirstlane(len[s]);
                    if (geo) g = __builtin_amdgcn_readfirstlane(geo[s]);
                    nt = seq_tiles(L, geo ? geo_ts(g) : 4);
                } while (nt == 0);
            }
        }
        int f = 0;
        if (!(wf & 1)) {                   // a new segment starts here
            f |= kFirst;
            wf = (wf & 4) | (tile == 0 ? 2 : 0);
        }
        if (wf & 4) f |= kSlot1;
        o.key = (s << 12) | h | (geo ? geo_code(g) << 25 : 0);
        o.L = L;
        o.t0 = tile;
        const int shift = geo ? geo_shift(g) : bs_shift, ts = geo ? geo_ts(g) : 4;
        o.wb = (tile << ts) >> shift;
        const int wend = ((o.wb + 64) << shift) >> ts;     // first tile past the window
        int t1 = min(nt, tile + rem);
        t1 = min(t1, wend);
        o.t1 = t1;
        o.chunk = chunk;
        rem -= t1 - tile;
        tile = t1;
        const bool last = (tile >= nt) || rem <= 0;
        if (last) {
            f |= kLast;
            if (wf & 2) f |= kStart;
            if (tile >= nt) f |= kEnd;
            if ((wf & 2) && tile >= nt) f |= kComplete;
            wf = 4;                        // closed; later segments use slot 1
        } else {
            wf |= 1;
        }
        o.flags = f;
        return true;
    }
};

// MULTI: speculative verification (several query tokens per sequence, at
// most 16 / G of them, query_start in p.q_start).  The last query token of a
// sequence sees all its L tokens, so the streams, chunks and walk are those
// of decode; the B operand's 16 columns are (query token, head) pairs as in
// multi_query.hip, each column drops the tokens past its own position, and
// rows and partial entries are per column (QPG * G of them per chunk slot).
// MIXED: block sizes per sequence over a pool of pages (p.bs tokens each,
// as decode_mixed_kernel): each sequence walks its own block size, and
// sequences of 8-token blocks walk 8-token tiles.
// KLDS: K tiles staged in LDS (TileMath); the ring's K slots follow the
// prefix arrays in LDS (ring_offset).
template <class Q, class C, int D, bool PAIR, int DEPTH, bool MULTI, bool MIXED, bool KLDS>
__global__ __launch_bounds__(64 * kWaves, 1) void decode_balanced_kernel(DecodeParams p) {
    static_assert(!(MULTI && MIXED) && !(PAIR && MIXED), "one mode at a time");
    typedef TileMath<Q, C, D, PAIR, KLDS> TM;
    typedef typename TM::T T;
    typedef typename TM::v8 v8;
    extern __shared__ int lds[];
    int* pre = lds;                        // [S + 1] tile prefix
    int* len = lds + p.S + 1;              // [S] clamped lengths
    int* qs = lds + 2 * p.S + 1;           // MULTI: [S + 1] query_start
    int* geo = lds + 2 * p.S + 1;          // MIXED: [S] geometries
    int32_t* hdr = p.ws_hdr;
    if constexpr (MULTI) {
        for (int i = threadIdx.x; i <= p.S; i += 64 * kWaves) qs[i] = p.q_start[i];
    }
    wg_prefix<MIXED>(p, pre, len, geo);

    const TM tm;
    const int lane = tm.lane;
    const int w = blockIdx.x * kWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // final chunks of at least two rounds of the ring
    const Sched q = make_sched(__builtin_amdgcn_readfirstlane(pre[p.S]), p.nW, 2 * DEPTH);
    if (blockIdx.x == 0) {
        // what the reduce needs: the prefix and the schedule
        for (int i = threadIdx.x; i <= p.S; i += 64 * kWaves) p.ws_pre[i] = pre[i];
        if (threadIdx.x == 0) {
            hdr[kHdrMagic] = kBalancedMagic;
            hdr[kHdrNW] = p.nW;
            hdr[kHdrHkv] = p.Hkv;
            hdr[kHdrG] = p.G;
            hdr[kHdrT] = q.T;
            hdr[kHdrC1] = q.C1;
            hdr[kHdrC2] = q.C2;
            hdr[kHdrC3] = q.C3;
            hdr[kHdrChunks] = q.chunks;
            hdr[kHdrFloor] = 2 * DEPTH;
        }
    }
    if (w >= q.chunks || w >= p.nW) return;
    const int G = p.G;
    const int bs_shift = p.bs == 8 ? 3 : (p.bs == 16 ? 4 : 5);
    const int* geo_s = MIXED ? geo : nullptr;             // per sequence, or
    const int geo0 = MIXED ? 0 : geo_pack(bs_shift, 4);  // the pool's (unread)
    unsigned long long* counter = (unsigned long long*)(hdr + kHdrCounter);
    const int QPG = MULTI ? 16 / G : 1;    // query tokens per stream
    const int ncol = QPG * G;              // columns (rows) per stream
    // MULTI: first query row and query tokens (at most QPG) of sequence s
    auto q_first = [&](int s) { return __builtin_amdgcn_readfirstlane(qs[s]); };
    auto q_count = [&](int s) {
        const int n = __builtin_amdgcn_readfirstlane(qs[s + 1]) - q_first(s);
        return max(0, min(n, QPG));
    };

    // ---- requests made one round ahead ---------------------------------
    // The index of the wave's next chunk (the counter's atomic add), the
    // table window of the producer's next span and the query rows of a
    // segment the producer enters are requested once per round, at the end
    // of the round, by instructions that run every round (out of range, so
    // touching nothing, when nothing is wanted), and taken one round later,
    // after the consumer has waited for the tiles issued before them.  A
    // result still in flight is never copied or branched around, which would
    // make the loop wait for every load in flight.
    const rsrc_t ctr = make_rsrc((const char*)counter, 8);
    long long got = 0;
    bool issued = false;                   // `got` is a chunk request in flight
    bool have = false;                     // `pend` holds an unused chunk index
    int pend = 0;
    bool chunks_left = true;
    // chunk index (counter-relative) from a value an add returned
    auto index_of = [&](long long v) {
        const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
        const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
        const uint64_t u = ((uint64_t)hi << 32) | lo;
        if (counter_live(u, p.epoch)) return (int)(lo & kCountMask);
        return counter_rebase(counter, p.epoch);
    };
    auto take_chunk = [&]() {
        int k;
        if (have) k = pend;
        else if (issued) k = index_of(got);
        else k = index_of(buffer_atomic_add_i64(1, ctr, lane == 0 ? 0 : (int)kOOB, 0, 0));
        have = issued = false;
        return q.nW + k;
    };

    // ---- producer: walks the wave's chunks one span ahead of the issue ----
    // Within a chunk the walk looks one span ahead; it steps into the next
    // chunk only once that chunk's index is at hand.
    Walk pw;
    pw.start(pre, len, geo_s, geo0, p.S, w, chunk_start<MULTI>(q, w, pre, len, geo_s, p.S),
             chunk_start<MULTI>(q, w + 1, pre, len, geo_s, p.S));
    auto walk_next = [&](Span& o) { return pw.next(len, geo_s, p.S, p.Hkv, bs_shift, o); };
    auto chunk_next = [&](Span& o) {       // first span of the next chunk
        const int c = take_chunk();
        if (c >= q.chunks) {
            chunks_left = false;
            return false;
        }
        pw.start(pre, len, geo_s, geo0, p.S, c, chunk_start<MULTI>(q, c, pre, len, geo_s, p.S),
                 chunk_start<MULTI>(q, c + 1, pre, len, geo_s, p.S));
        return walk_next(o);               // chunks are never empty
    };
    // Window of 64 block-table entries from block sp.wb; entries at or past
    // ceil(L / bs) are outside the descriptor and read 0 (never touched).
    auto load_window = [&](const Span& sp, bool want) {
        int nblk;
        if constexpr (MIXED) {
            const int sh = code_shift(sp.code());
            nblk = want ? (sp.L + (1 << sh) - 1) >> sh : 0;
        } else {
            nblk = want ? (sp.L + p.bs - 1) >> bs_shift : 0;
        }
        const rsrc_t r = make_rsrc((const char*)(p.tables + (size_t)sp.template seq<MIXED>() * p.max_blocks),
                                   (uint32_t)nblk * 4u);
        return (int)Buf<4>::load(r, (uint32_t)(sp.wb + lane) * 4u);
    };
    // MULTI: column j16 is head j16 % G of query token j16 / G; its offset
    // from the token group's first row, and the first query row and token
    // count of the producer's sequence (kept beside its span, so the
    // per-round request reads no LDS).
    const int col_tok = MULTI ? tm.j16 / G : 0;
    const uint32_t col_off =
        MULTI ? (uint32_t)((col_tok * p.Hq + tm.j16 % G) * D * sizeof(T)) : 0u;
    int ps_q0 = 0, ps_n = 0;
    // Query rows of the span's group as the B operand (heads past G read 0).
    auto load_query = [&](const Span& sp, bool want, v8 (&qv)[TM::KS]) {
        size_t first_row = (size_t)sp.template seq<MIXED>();
        uint32_t range = (uint32_t)(G * D * sizeof(T));
        uint32_t row = (uint32_t)(tm.j16 * D * sizeof(T));
        if constexpr (MULTI) {
            first_row = (size_t)ps_q0;
            range = ps_n > 0 ? (uint32_t)(((ps_n - 1) * p.Hq + G) * D * sizeof(T)) : 0u;
            row = col_tok < ps_n ? col_off : kOOB;
        }
        const char* base = (const char*)p.q + (first_row * p.Hq + (size_t)sp.h() * G) * D * sizeof(T);
        const rsrc_t r = make_rsrc(base, want ? range : 0u);
#pragma unroll
        for (int kk = 0; kk < TM::KS; kk++) {
            const int d0 = TM::kFp8 ? (kk >> 1) * 64 + 16 * tm.g4 + (kk & 1) * 8 : 32 * kk + 8 * tm.g4;
            qv[kk] = __builtin_bit_cast(v8, Buf<16>::load(r, row + (uint32_t)(d0 * sizeof(T))));
        }
    };

    Span ps, pn;
    walk_next(ps);                         // chunk w is not empty
    if constexpr (MULTI) {
        ps_q0 = q_first(ps.template seq<MIXED>());
        ps_n = q_count(ps.template seq<MIXED>());
    }
    v8 qb[TM::KS];                         // query of the consumer's segment
    load_query(ps, true, qb);
    int win = load_window(ps, true);
    bool has_ps = true;
    bool has_pn = walk_next(pn);
    int win_n = load_window(pn, has_pn);   // window of pn
    // K/V of the span's stream; MIXED: blocks of the sequence's size, each
    // (1 << shift) / p.bs consecutive pages from the page its entry names
    auto head_of = [&](const Span& sp) {
        Head hd = make_head<C, D>(p, sp.h());
        if constexpr (MIXED) {
            const int sh = code_shift(sp.code());
            hd.bs_shift = sh;
            hd.rec_bytes = (hd.row_bytes << sh) - (uint32_t)(sp.h() * D * C::kBytes);
            hd.nb_last = (uint32_t)(p.NB - (1 << (sh - p.page_shift)));
        }
        return hd;
    };
    Head hd = head_of(ps);
    int prt = ps.t0;

    bool want_win = false, want_q = false;  // set when pn / ps change
    // Producer's step to the round after the one just issued.
    auto producer_advance = [&]() {
        prt += DEPTH;
        if (has_ps && prt >= ps.t1) {
            if (!has_pn && chunks_left) {
                // the next chunk's index is late: wait for it and its window
                has_pn = chunk_next(pn);
                if (has_pn) win_n = settled(load_window(pn, true));
            }
            has_ps = has_pn;
            if (has_ps) {
                ps = pn;
                if constexpr (MULTI) {
                    ps_q0 = q_first(ps.template seq<MIXED>());
                    ps_n = q_count(ps.template seq<MIXED>());
                }
                win = win_n;
                prt = ps.t0;
                hd = head_of(ps);
                want_q = (ps.flags & kFirst) != 0;
                has_pn = walk_next(pn);
                want_win = has_pn;
            }
        }
        if (has_ps && !has_pn && have) {   // look ahead into the next chunk
            has_pn = chunk_next(pn);
            want_win = has_pn;
        }
    };
    int wload;                              // window requested this round
    v8 qload[TM::KS];                       // query requested this round
    // End of a round: the requests.
    auto request = [&]() {
        // The next chunk's index is requested when the walk has reached the
        // end of the current chunk and fewer than kRequestAhead of its tiles
        // are left to issue: early enough to arrive in time, late enough
        // that waves (which start together) ask at different times.
        const int left = (ps.t1 - prt) + (has_pn ? pn.t1 - pn.t0 : 0);
        const bool want = !have && !issued && chunks_left && has_ps && pw.rem <= 0 &&
                          left < kRequestAhead;
        got = buffer_atomic_add_i64(1, ctr, lane == 0 && want ? 0 : (int)kOOB, 0, 0);
        issued = want;
        wload = load_window(pn, want_win);
        load_query(ps, want_q, qload);
    };
    // One round later: take them.  `got` must be taken before the next
    // request, which reuses it.
    auto take_chunk_index = [&]() {
        if (issued) {
            pend = index_of(got);
            have = true;
            issued = false;
        }
    };
    auto take = [&]() {
        take_chunk_index();
        if (want_win) {
            win_n = wload;
            want_win = false;
        }
    };

    // ---- consumer: one round behind, on the producer's previous span ------
    typename TM::Tile tl[DEPTH];
    // KLDS: this wave's K slots, one per ring buffer
    lds_t* const kring =
        (lds_t*)((char*)lds + ring_offset(p.S, MULTI || MIXED)) +
        (size_t)__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) * DEPTH * TM::kKSlot;
    auto kslot = [&](int j) { return kring + j * TM::kKSlot; };
#pragma unroll
    for (int j = 0; j < DEPTH; j++) {
        const int tp = prt + j;
        if constexpr (MIXED) {
            const int ts = code_ts(ps.key >> 25);
            tm.issue(hd, tp << ts, tp < ps.t1 ? min(ps.L - 1 - (tp << ts), (1 << ts) - 1) : -1,
                     ps.wb, win, tl[j], kslot(j));
        } else
            tm.issue(hd, tp << 4, tp < ps.t1 ? ps.L - 1 - (tp << 4) : -1, ps.wb, win, tl[j],
                     kslot(j));
        if constexpr (KLDS) __builtin_amdgcn_sched_barrier(0);
    }
    // consumer's span: its stream, length, end tile, chunk and flags
    int c_key = ps.key, c_L = ps.L, c_t1 = ps.t1, c_chunk = ps.chunk, c_flags = ps.flags;
    int c_ts = MIXED ? code_ts(ps.key >> 25) : 4;   // log2 of the consumer's tile
    int crt = ps.t0;
    // MULTI: this lane's column's last visible token in the consumer's
    // sequence (-1: none)
    auto column_limit = [&](int s, int L) {
        const int n = q_count(s);
        return col_tok < n ? L - n + col_tok : -1;
    };
    int c_pc = MULTI ? column_limit(c_key >> 12, c_L) : 0;
    typename TM::Acc acc;
    tm.reset(acc);
    producer_advance();
    request();

    while (true) {
#pragma unroll
        for (int j = 0; j < DEPTH; j++) {
            const int tc = crt + j;
            if constexpr (KLDS) {
                // Slot j's K loads are done once at most the loads of the
                // DEPTH - 1 tiles issued after them are in flight (every
                // round issues all DEPTH tiles, dead ones included, in ring
                // order; the round's requests and the tile's own V loads
                // only add to the count, so this may wait a little early).
                vm_wait<(DEPTH - 1) * TM::kLoadsPerTile>();
                __builtin_amdgcn_sched_barrier(0);
            }
            if (j == 0 || tc < c_t1) {
                if constexpr (MULTI)
                    tm.template consume<true>(acc, qb, p.scale_log2, c_L - 1 - (tc << 4), tl[j],
                                              c_pc - (tc << 4), kslot(j));
                else
                    tm.consume(acc, qb, p.scale_log2,
                               MIXED ? min(c_L - 1 - (tc << c_ts), (1 << c_ts) - 1)
                                     : c_L - 1 - (tc << 4),
                               tl[j], 0, kslot(j));
            }
            if constexpr (KLDS) __builtin_amdgcn_sched_barrier(0);
            const int tp = prt + j;
            if constexpr (MIXED) {
                const int ts = code_ts(ps.key >> 25);
                const int plim =
                    has_ps && tp < ps.t1 ? min(ps.L - 1 - (tp << ts), (1 << ts) - 1) : -1;
                tm.issue(hd, tp << ts, plim, ps.wb, win, tl[j], kslot(j));
            } else {
                const int plim = has_ps && tp < ps.t1 ? ps.L - 1 - (tp << 4) : -1;
                tm.issue(hd, tp << 4, plim, ps.wb, win, tl[j], kslot(j));
            }
            if constexpr (KLDS) __builtin_amdgcn_sched_barrier(0);
        }
        take();
        // Consumer first: finish its span and take the producer's current
        // one (the span of the round just issued) before the producer moves.
        crt += DEPTH;
        if (crt >= c_t1) {
            if (c_flags & kLast) {
                // the stream's chunk range, for the reduce: the segment that
                // starts the stream gives the first chunk and its slot there,
                // the one that ends it the last
                if (lane == 0 && (c_flags & (kStart | kEnd))) {
                    int32_t* rng = p.ws_pre + p.S + 1 +
                                   2 * ((MIXED ? (c_key >> 12) & 0x1FFF : c_key >> 12) * p.Hkv +
                                        (c_key & 4095));
                    if (c_flags & kStart)
                        rng[0] = c_chunk | ((c_flags & kSlot1) ? (int32_t)0x80000000 : 0);
                    if (c_flags & kEnd) rng[1] = c_chunk;
                }
                const size_t e0 = ((size_t)c_chunk * 2 + ((c_flags & kSlot1) ? 1 : 0)) * ncol;
                if constexpr (MULTI) {
                    const int cs = c_key >> 12, ch = c_key & 4095;
                    const size_t r0 = (size_t)q_first(cs);
                    const bool complete = (c_flags & kComplete) != 0;
                    tm.template finish_each<true>(
                        acc, q_count(cs) * G, [&](int) { return complete; }, p.v_scale,
                        [&](int c) {
                            return (T*)p.out + ((r0 + c / G) * p.Hq + (size_t)ch * G + c % G) * D;
                        },
                        [&](int c) { return p.ws_m + e0 + c; },
                        [&](int c) { return p.ws_l + e0 + c; },
                        [&](int c) { return (_Float16*)p.ws_o + (e0 + c) * D; });
                } else {
                    const size_t row0 =
                        (size_t)(MIXED ? (c_key >> 12) & 0x1FFF : c_key >> 12) * p.Hq +
                        (size_t)(c_key & 4095) * G;
                    tm.finish(
                        acc, G, (c_flags & kComplete) != 0, p.v_scale,
                        [&](int head) { return (T*)p.out + (row0 + head) * D; },
                        [&](int head) { return p.ws_m + e0 + head; },
                        [&](int head) { return p.ws_l + e0 + head; },
                        [&](int head) { return p.ws_o + (e0 + head) * D; });
                }
            }
            if (!has_ps) break;
            c_key = ps.key;
            c_L = ps.L;
            c_t1 = ps.t1;
            c_chunk = ps.chunk;
            c_flags = ps.flags;
            if constexpr (MIXED) c_ts = code_ts(ps.key >> 25);
            crt = ps.t0;
            if constexpr (MULTI) c_pc = column_limit(c_key >> 12, c_L);
            if (c_flags & kFirst) {
                // requested when the producer entered this segment
#pragma unroll
                for (int k = 0; k < TM::KS; k++) qb[k] = qload[k];
                tm.reset(acc);
            }
        }
        want_q = false;
        producer_advance();
        request();
    }
    // The ring's last round (dead tiles, zeros) may still be landing in the
    // K slots: let it land before the workgroup's LDS is handed on.
    if constexpr (KLDS) vm_wait<0>();
}

// One wavefront per SIMD, with deep rings.  Two waves on one SIMD do not
// stream at one rate: on MI355X the second-placed wave of each SIMD moved
// its tiles at half the rate of the first (per-wave timestamps), so the
// grid's ending was set by slow waves' last chunks.  One wave per SIMD with
// twice the tiles in flight (its ring spills into the accumulation
// registers, which cost a move, not memory traffic) removes the imbalance
// and keeps as many bytes in flight per SIMD: about 6% faster per call on
// the ragged GQA batch and 11% on long contexts.  An fp8 tile takes half the
// registers of a 16-bit one.
template <class C, int D, bool PAIR>
constexpr int pipeline_depth() {
    if (C::kBytes == 1) return PAIR ? 5 : 10;
    return PAIR ? 4 : (D == 64 ? 8 : 6);
}

// LDS of one compute unit (gfx950).
constexpr size_t kLdsPerCu = 160 * 1024;

template <class Q, class C, int D, bool PAIR>
hipError_t launch_k(const DecodeParams& p, hipStream_t st) {
    const dim3 grid((unsigned)((p.nW + kWaves - 1) / kWaves)), block(64 * kWaves);
    void* args[] = {const_cast<DecodeParams*>(&p)};
    constexpr int DP = pipeline_depth<C, D, PAIR>();
    const bool multi = p.q_start != nullptr;
    const bool mixed = p.seq_bs != nullptr;
    // K staged in LDS where the ring's slots fit beside the prefix arrays
    constexpr size_t ring = (size_t)kWaves * DP * TileMath<Q, C, D, false, true>::kKSlot;
    const size_t lds_k = ring_offset(p.S, multi || mixed) + ring;
    // (8-token blocks of a uniform pool take the two-block PAIR tile; its K
    // goes through LDS too where each row-order load lies in one block, that
    // is with at most 8 rows per load)
    constexpr bool can = !PAIR || 1024 / (D * C::kBytes) <= 8;
    const bool klds = can && lds_k <= kLdsPerCu;
    const void* k = nullptr;
    if constexpr (PAIR) {
        if constexpr (can) {
            if (klds) {
                k = multi ? reinterpret_cast<const void*>(decode_balanced_kernel<Q, C, D, true, DP, true, false, true>)
                          : reinterpret_cast<const void*>(decode_balanced_kernel<Q, C, D, true, DP, false, false, true>);
                return hipLaunchKernel(k, grid, block, args, lds_k, st);
            }
        }
        k = multi ? reinterpret_cast<const void*>(decode_balanced_kernel<Q, C, D, true, DP, true, false, false>)
                  : reinterpret_cast<const void*>(decode_balanced_kernel<Q, C, D, true, DP, false, false, false>);
    } else if (multi) {
        k = klds ? reinterpret_cast<const void*>(decode_balanced_kernel<Q, C, D, false, DP, true, false, true>)
                 : reinterpret_cast<const void*>(decode_balanced_kernel<Q, C, D, false, DP, true, false, false>);
    } else if (mixed) {
        k = klds ? reinterpret_cast<const void*>(decode_balanced_kernel<Q, C, D, false, DP, false, true, true>)
                 : reinterpret_cast<const void*>(decode_balanced_kernel<Q, C, D, false, DP, false, true, false>);
    } else {
        k = klds ? reinterpret_cast<const void*>(decode_balanced_kernel<Q, C, D, false, DP, false, false, true>)
                 : reinterpret_cast<const void*>(decode_balanced_kernel<Q, C, D, false, DP, false, false, false>);
    }
    return hipLaunchKernel(k, grid, block, args, klds ? lds_k : lds_bytes(p.S, multi || mixed), st);
}

template <class Q, class C, int D, bool PAIR>
int resident_k(int S) {
    int blocks = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &blocks, decode_balanced_kernel<Q, C, D, PAIR, pipeline_depth<C, D, PAIR>(), false, false, false>,
            64 * kWaves, lds_bytes(S, true)) != hipSuccess)
        return 0;
    // one workgroup per CU = one wavefront per SIMD, also where the
    // registers would hold two (head_dim 64)
    return (blocks < 1 ? blocks : 1) * kWaves;
}

template <class Q, class C>
hipError_t launch_d(const DecodeParams& p, hipStream_t st) {
    const bool pair = p.bs == 8 && p.seq_bs == nullptr;   // mixed sizes take 8-token tiles
    if (p.D == 64) return pair ? launch_k<Q, C, 64, true>(p, st) : launch_k<Q, C, 64, false>(p, st);
    if (p.D == 128)
        return pair ? launch_k<Q, C, 128, true>(p, st) : launch_k<Q, C, 128, false>(p, st);
    return hipErrorInvalidValue;
}

template <class Q, class C>
int resident_d(int D, int bs, int S) {
    const bool pair = bs == 8;
    if (D == 64) return pair ? resident_k<Q, C, 64, true>(S) : resident_k<Q, C, 64, false>(S);
    if (D == 128) return pair ? resident_k<Q, C, 128, true>(S) : resident_k<Q, C, 128, false>(S);
    return 0;
}

}  // namespace

int decode_balanced_waves_per_cu(int qdt, int cdt, int D, int bs, int S) {
    if (qdt == kBF16)
        return cdt == kFP8 ? resident_d<BF16, FP8>(D, bs, S) : resident_d<BF16, BF16>(D, bs, S);
    if (qdt == kF16)
        return cdt == kFP8 ? resident_d<F16, FP8>(D, bs, S) : resident_d<F16, F16>(D, bs, S);
    return 0;
}

hipError_t launch_decode_balanced(int qdt, int cdt, const DecodeParams& p, hipStream_t st) {
    if (!decode_mfma_supported(qdt, cdt, p.D, p.G)) return hipErrorInvalidValue;
    if (p.S > kBalancedMaxSeqs || p.nW < 1 || p.nW > kBalancedMaxWaves) return hipErrorInvalidValue;
    if (qdt == kBF16) {
        if (cdt == kFP8) return launch_d<BF16, FP8>(p, st);
        return launch_d<BF16, BF16>(p, st);
    }
    if (cdt == kFP8) return launch_d<F16, FP8>(p, st);
    return launch_d<F16, F16>(p, st);
}

}  // namespace pkv
