// api.hip - the C ABI of libpagedkv (declared in include/pagedkv.h).
//
// Host-side argument validation, workspace layout and kernel dispatch.  No
// call allocates, frees or synchronises; every error is returned before
// anything is enqueued.
#include "pagedkv.h"

#include <atomic>
#include <chrono>

#include "common.hpp"
#include "kernels.hpp"

namespace {

using namespace pkv;

// Numbers the balanced decode calls of the process.  A call tells the
// chunk-counter state left in its workspace by an earlier call from its own
// by this number (kernels.hpp), so numbers must not repeat for a long time:
// a 32-bit sequence, started from the clock.
uint32_t next_call_number() {
    static std::atomic<uint32_t> next{
        (uint32_t)std::chrono::steady_clock::now().time_since_epoch().count()};
    return next.fetch_add(1, std::memory_order_relaxed);
}

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

inline bool valid_dtype(int d) { return d >= PKV_F32 && d <= PKV_FP8_E4M3; }

inline int elem_bytes(int d) { return d == PKV_F32 ? 4 : (d == PKV_FP8_E4M3 ? 1 : 2); }

inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Workspace pieces for split-K.  Fixed partitions: P_max entries per row,
// m at 0, l at off_l, o at off_o.  Balanced: a 256-byte header, the tile
// prefix of the sequences (S + 1 words) at off_pre followed by the chunk
// range of each (sequence, KV head) stream (2 words each), then m, l and o
// for two entries per query head of the group per chunk of the guided
// schedule, sized for the largest grid (kBalancedMaxWaves) and its chunk
// bound.
struct WsLayout {
    int P_max = 0;
    size_t off_pre = 0, off_m = 0, off_l = 0, off_o = 0, bytes = 0;
};

inline bool ws_layout(int32_t S, int32_t Hq, int32_t Hkv, int32_t D, int32_t max_seq_len,
                      int32_t P, WsLayout* w) {
    if (S <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || max_seq_len <= 0 || Hq % Hkv != 0)
        return false;
    size_t n;
    if (P == PKV_PARTITION_BALANCED) {
        w->P_max = 0;
        w->off_pre = 256;
        w->off_m = round_up(w->off_pre + 4 * ((size_t)S + 1) + 8 * (size_t)S * (size_t)Hkv, 256);
        n = (size_t)2 * (size_t)max_chunks(kBalancedMaxWaves) * (size_t)(Hq / Hkv);
    } else {
        if (P <= 0) return false;
        w->P_max = (int)((max_seq_len + (int64_t)P - 1) / P);
        w->off_m = 0;
        n = (size_t)S * (size_t)Hq * (size_t)w->P_max;
    }
    w->off_l = w->off_m + round_up(n * 4, 256);
    w->off_o = w->off_l + round_up(n * 4, 256);
    w->bytes = w->off_o + n * (size_t)D * 4;
    return true;
}

// Resident wavefronts of the whole device for the balanced kernel serving
// these types and shapes, capped at kBalancedMaxWaves.  The CU count and the
// kernel's occupancy are asked once per device and kernel variant (with the
// largest LDS the kernel takes, so the answer holds for every batch size)
// and kept for the life of the process; a call then costs one hipGetDevice.
constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];                 // 0: not asked yet
std::atomic<int> g_per_cu[kMaxDevices][2][2][2][3];  // [q f16/bf16][cache 16-bit/fp8][D][bs]

inline int balanced_grid_waves(int qdt, int cdt, int D, int bs) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = -1;
    const bool cached = dev >= 0 && dev < kMaxDevices;
    int cus = cached ? g_cus[dev].load(std::memory_order_relaxed) : 0;
    if (cus <= 0) {
        if (dev < 0 ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus <= 0)
            cus = 256;
        if (cached) g_cus[dev].store(cus, std::memory_order_relaxed);
    }
    std::atomic<int>* slot =
        cached ? &g_per_cu[dev][qdt == PKV_BF16][cdt == PKV_FP8_E4M3][D == 128]
                          [bs == 8 ? 0 : (bs == 16 ? 1 : 2)]
               : nullptr;
    int per_cu = slot ? slot->load(std::memory_order_relaxed) : 0;
    if (per_cu <= 0) {
        per_cu = decode_balanced_waves_per_cu(qdt, cdt, D, bs, kBalancedMaxSeqs);
        if (per_cu <= 0) per_cu = 4;
        if (slot) slot->store(per_cu, std::memory_order_relaxed);
    }
    const long n = (long)cus * per_cu;
    return (int)(n < kBalancedMaxWaves ? n : kBalancedMaxWaves);
}

inline bool supported_block_size(int32_t bs) { return bs == 8 || bs == 16 || bs == 32; }

inline bool valid_decode_types(int qdt, int cdt) {
    if (qdt == PKV_FP8_E4M3) return false;
    if (cdt == PKV_FP8_E4M3) return qdt == PKV_F16 || qdt == PKV_BF16;
    return qdt == cdt;
}

// Multi-query split-K workspace: m, l [rows][P_max], o [rows][P_max][D] for
// rows = num_seqs * max_query_len * num_q_heads (the bound on query rows),
// then the per-query-token lengths [num_seqs * max_query_len] int32.
struct MultiWs {
    int P_max = 1;
    size_t off_m = 0, off_l = 0, off_o = 0, off_len = 0, bytes = 0;
};

inline bool multi_ws_layout(int S, int Qmax, int Hq, int D, int max_len, int P, MultiWs* w) {
    if (S <= 0 || Qmax <= 0 || Hq <= 0 || D <= 0 || max_len <= 0) return false;
    if (P == 0) return true;
    if (P == PKV_PARTITION_BALANCED) {
        // the balanced layout: header, tile prefix and stream chunk ranges
        // (for up to Hq KV heads), then entries of 16 columns (query token,
        // head) per chunk slot
        auto up = [](int64_t x) { return (x + 255) / 256 * 256; };
        const int64_t n = 2 * max_chunks(kBalancedMaxWaves) * 16;
        w->P_max = 1;
        w->off_len = 256;                          // the tile prefix here
        w->off_m = (size_t)up(256 + 4 * ((int64_t)S + 1) + 8 * (int64_t)S * Hq);
        w->off_l = w->off_m + (size_t)up(4 * n);
        w->off_o = w->off_l + (size_t)up(4 * n);
        w->bytes = w->off_o + (size_t)(4 * n * D);
        return true;
    }
    if (P < 0) return false;
    w->P_max = (int)(((int64_t)max_len + P - 1) / P);
    const int64_t rows = (int64_t)S * Qmax * Hq;
    const int64_t n = rows * w->P_max;
    if (n * D > ((int64_t)1 << 31) || (int64_t)S * Qmax > ((int64_t)1 << 30)) return false;
    auto up = [](int64_t x) { return (x + 255) / 256 * 256; };
    w->off_m = 0;
    w->off_l = (size_t)up(4 * n);
    w->off_o = 2 * w->off_l;
    w->off_len = w->off_o + (size_t)up(4 * n * D);
    w->bytes = w->off_len + (size_t)up(4 * (int64_t)S * Qmax);
    return true;
}

inline int launch_status(hipError_t e) { return e == hipSuccess ? PKV_OK : PKV_ERR_HIP; }

// The group size of a reduce's rows and its log2 (-1 when not a power of 2).
inline void set_group(ReduceParams& r) {
    r.G = r.Hq / r.Hkv;
    r.g_shift = (r.G & (r.G - 1)) == 0 ? __builtin_ctz((unsigned)r.G) : -1;
}

}  // namespace

extern "C" {

const char* pkv_status_string(int status) {
    switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_NULL: return "a required pointer is NULL";
    case PKV_ERR_SHAPE: return "a size is out of range or inconsistent";
    case PKV_ERR_DTYPE: return "unknown dtype or invalid dtype pairing";
    case PKV_ERR_UNSUPPORTED: return "no kernel for this combination";
    case PKV_ERR_WORKSPACE: return "workspace missing or too small";
    case PKV_ERR_ALIGN: return "a device pointer is not 16-byte aligned";
    case PKV_ERR_HIP: return "HIP launch error";
    case PKV_ERR_NO_BLOCKS: return "no free block in the pool";
    case PKV_ERR_SCRATCH: return "the call needs more than the library's fixed scratch array";
    default: return "unknown status";
    }
}

int pkv_reshape_and_cache(const void* key, const void* value, pkv_dtype src_dtype,
                          void* k_cache, void* v_cache, pkv_dtype cache_dtype,
                          const int64_t* slot_mapping, int32_t num_tokens,
                          int32_t num_kv_heads, int32_t head_dim,
                          int32_t block_size, int32_t num_blocks, float k_scale,
                          float v_scale, hipStream_t stream) {
    if (!valid_dtype(src_dtype) || !valid_dtype(cache_dtype)) return PKV_ERR_DTYPE;
    if (src_dtype == PKV_FP8_E4M3) return PKV_ERR_DTYPE;
    if (cache_dtype != src_dtype && cache_dtype != PKV_FP8_E4M3) return PKV_ERR_DTYPE;
    if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
        num_blocks <= 0)
        return PKV_ERR_SHAPE;
    if (head_dim % 8 != 0) return PKV_ERR_UNSUPPORTED;
    if (cache_dtype == PKV_FP8_E4M3 &&
        !(k_scale > 0.0f && v_scale > 0.0f && k_scale < INFINITY && v_scale < INFINITY))
        return PKV_ERR_SHAPE;
    if (num_tokens == 0) return PKV_OK;
    if (!key || !value || !k_cache || !v_cache || !slot_mapping) return PKV_ERR_NULL;
    if (!aligned16(key) || !aligned16(value) || !aligned16(k_cache) || !aligned16(v_cache) ||
        ((uintptr_t)slot_mapping & 7u))
        return PKV_ERR_ALIGN;
    WriteParams p;
    p.key = key;
    p.value = value;
    p.k_cache = k_cache;
    p.v_cache = v_cache;
    p.slot_mapping = slot_mapping;
    p.num_slots = (int64_t)num_blocks * block_size;
    p.T = num_tokens;
    p.Hkv = num_kv_heads;
    p.D = head_dim;
    p.src_bytes = src_dtype == PKV_F32 ? 4 : 2;
    p.k_scale = k_scale;
    p.v_scale = v_scale;
    return launch_status(launch_reshape_and_cache(src_dtype, cache_dtype, p, stream));
}

int pkv_paged_attention_multi(void* out, const void* query, pkv_dtype q_dtype,
                              const void* k_cache, const void* v_cache,
                              pkv_dtype cache_dtype, const int32_t* block_tables,
                              int32_t max_blocks_per_seq, const int32_t* seq_lens,
                              const int32_t* query_start, int32_t num_seqs,
                              int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                              int32_t block_size, int32_t num_blocks, int32_t max_seq_len,
                              int32_t max_query_len, float scale, float k_scale,
                              float v_scale, int32_t partition_size, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
    if (!valid_dtype(q_dtype) || !valid_dtype(cache_dtype)) return PKV_ERR_DTYPE;
    if (!valid_decode_types(q_dtype, cache_dtype)) return PKV_ERR_DTYPE;
    if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        block_size <= 0 || num_blocks <= 0 || max_blocks_per_seq <= 0 || max_seq_len <= 0 ||
        max_query_len <= 0 || (partition_size < 0 && partition_size != PKV_PARTITION_BALANCED))
        return PKV_ERR_SHAPE;
    if (num_q_heads % num_kv_heads != 0) return PKV_ERR_SHAPE;
    if (num_kv_heads > 4096) return PKV_ERR_SHAPE;
    if (!(scale == scale) || !(k_scale == k_scale) || !(v_scale == v_scale)) return PKV_ERR_SHAPE;
    if (!supported_block_size(block_size)) return PKV_ERR_UNSUPPORTED;
    if (partition_size > 0 && (partition_size % 16 != 0 || partition_size % block_size != 0))
        return PKV_ERR_SHAPE;
    const int G = num_q_heads / num_kv_heads;
    if (!decode_mfma_supported(q_dtype, cache_dtype, head_dim, G)) return PKV_ERR_UNSUPPORTED;
    if (!out || !query || !k_cache || !v_cache || !block_tables || !seq_lens || !query_start)
        return PKV_ERR_NULL;
    if (!aligned16(out) || !aligned16(query) || !aligned16(k_cache) || !aligned16(v_cache) ||
        ((uintptr_t)block_tables & 3u) || ((uintptr_t)seq_lens & 3u) ||
        ((uintptr_t)query_start & 3u))
        return PKV_ERR_ALIGN;
    const int qpg = 16 / G;                        // query tokens per column block
    // long query runs without a split: 2 or 4 column blocks per wavefront
    const int nb = partition_size != 0 || max_query_len <= qpg ? 1
                   : (max_query_len >= 4 * qpg ? 4 : 2);
    // runs of at least 64 / G tokens (two wavefronts' rows) of 16-bit
    // queries and caches: the LDS-staged kernel
    const int ptok = prefill_tokens_per_group(G);
    const bool staged = partition_size == 0 && G * max_query_len >= 64 &&
                        prefill_supported(q_dtype, cache_dtype, head_dim, G);
    const int64_t groups =
        staged ? (max_query_len + (int64_t)ptok - 1) / ptok
               : (max_query_len + (int64_t)qpg * nb - 1) / ((int64_t)qpg * nb);
    const int64_t cap = (int64_t)max_blocks_per_seq * block_size;
    const int len_cap = (int)(cap < max_seq_len ? cap : max_seq_len);
    MultiWs w;
    if (!multi_ws_layout(num_seqs, max_query_len, num_q_heads, head_dim, len_cap,
                         partition_size, &w))
        return PKV_ERR_SHAPE;
    const int64_t units = (int64_t)num_seqs * w.P_max * groups * num_kv_heads;
    if (units > ((int64_t)1 << 31) - 64) return PKV_ERR_SHAPE;
    const bool balanced = partition_size == PKV_PARTITION_BALANCED;
    if (balanced) {
        // one column group of 16 / G query tokens per sequence; tile counts
        // are 32-bit on the device
        if (max_query_len > qpg || num_seqs > kBalancedMaxSeqs) return PKV_ERR_UNSUPPORTED;
        const int64_t tiles = (int64_t)num_seqs * num_kv_heads * ((len_cap + 15) / 16);
        if (tiles > ((int64_t)1 << 31) - 1) return PKV_ERR_SHAPE;
    }
    if (partition_size != 0) {
        if (!workspace || workspace_bytes < w.bytes) return PKV_ERR_WORKSPACE;
        if (!aligned16(workspace)) return PKV_ERR_ALIGN;
    }

    DecodeParams p;
    p.out = out;
    p.q = query;
    p.k = k_cache;
    p.v = v_cache;
    p.tables = block_tables;
    p.lens = seq_lens;
    p.ws_m = p.ws_l = p.ws_o = nullptr;
    p.ws_hdr = p.ws_pre = nullptr;
    p.nW = 0;
    p.epoch = 0;
    p.q_start = query_start;
    p.max_groups = (int)groups;
    p.col_blocks = nb;
    p.ws_len = nullptr;
    p.len_rows = num_seqs * max_query_len;
    p.seq_bs = nullptr;
    p.page_shift = 0;
    p.S = num_seqs;
    p.Hq = num_q_heads;
    p.Hkv = num_kv_heads;
    p.D = head_dim;
    p.G = G;
    p.bs = block_size;
    p.NB = num_blocks;
    p.max_blocks = max_blocks_per_seq;
    p.len_cap = len_cap;
    p.P = partition_size;
    p.P_max = w.P_max;
    const float ks = cache_dtype == PKV_FP8_E4M3 ? k_scale : 1.0f;
    p.scale_log2 = scale * ks * kLog2e;
    p.v_scale = cache_dtype == PKV_FP8_E4M3 ? v_scale : 1.0f;
    if (balanced) {
        p.P = 0;
        p.P_max = 1;
        p.ws_hdr = (int32_t*)workspace;
        p.ws_pre = (int32_t*)((char*)workspace + w.off_len);
        p.ws_m = (float*)((char*)workspace + w.off_m);
        p.ws_l = (float*)((char*)workspace + w.off_l);
        p.ws_o = (float*)((char*)workspace + w.off_o);
        p.nW = balanced_grid_waves(q_dtype, cache_dtype, head_dim, block_size);
        p.epoch = next_call_number();
        hipError_t e = launch_decode_balanced(q_dtype, cache_dtype, p, stream);
        if (e != hipSuccess) return launch_status(e);
        ReduceParams r;
        r.out = out;
        r.ws_hdr = p.ws_hdr;
        r.ws_pre = p.ws_pre;
        r.ws_m = p.ws_m;
        r.ws_l = p.ws_l;
        r.ws_o = p.ws_o;
        r.lens = seq_lens;
        r.S = p.len_rows;
        r.Hq = num_q_heads;
        r.Hkv = num_kv_heads;
        r.D = head_dim;
        r.P = 0;
        r.P_max = 1;
        r.len_cap = len_cap;
        r.q_start = query_start;
        r.S_seq = num_seqs;
        set_group(r);
        return launch_status(launch_reduce_balanced(q_dtype, r, stream));
    }
    if (partition_size > 0) {
        p.ws_m = (float*)((char*)workspace + w.off_m);
        p.ws_l = (float*)((char*)workspace + w.off_l);
        p.ws_o = (float*)((char*)workspace + w.off_o);
        p.ws_len = (int32_t*)((char*)workspace + w.off_len);
    }
    if (staged) return launch_status(launch_prefill(q_dtype, cache_dtype, p, stream));
    hipError_t e = launch_multi_query(q_dtype, cache_dtype, p, stream);
    if (e != hipSuccess || partition_size == 0) return launch_status(e);
    // merge the partials of the rows (query token, query head)
    ReduceParams r;
    r.out = out;
    r.ws_m = p.ws_m;
    r.ws_l = p.ws_l;
    r.ws_o = p.ws_o;
    r.ws_hdr = r.ws_pre = nullptr;
    r.lens = p.ws_len;
    r.S = p.len_rows;
    r.Hq = num_q_heads;
    r.Hkv = num_kv_heads;
    r.D = head_dim;
    r.P = partition_size;
    r.P_max = w.P_max;
    r.len_cap = len_cap;
    r.q_start = nullptr;
    r.S_seq = num_seqs;
    return launch_status(launch_reduce(q_dtype, r, stream));
}

size_t pkv_multi_workspace_bytes(int32_t num_seqs, int32_t max_query_len, int32_t num_q_heads,
                                 int32_t head_dim, int32_t max_seq_len, int32_t partition_size) {
    if (partition_size <= 0 && partition_size != PKV_PARTITION_BALANCED) return 0;
    MultiWs w;
    if (!multi_ws_layout(num_seqs, max_query_len, num_q_heads, head_dim, max_seq_len,
                         partition_size, &w))
        return 0;
    return w.bytes;
}

int pkv_copy_blocks(void* dst_k, void* dst_v, const void* src_k, const void* src_v,
                    pkv_dtype cache_dtype, const int32_t* block_pairs, int32_t num_pairs,
                    int32_t src_blocks, int32_t dst_blocks, int32_t block_size,
                    int32_t num_kv_heads, int32_t head_dim, hipStream_t stream) {
    if (!valid_dtype(cache_dtype)) return PKV_ERR_DTYPE;
    if (num_pairs < 0 || src_blocks <= 0 || dst_blocks <= 0 || block_size <= 0 ||
        num_kv_heads <= 0 || head_dim <= 0)
        return PKV_ERR_SHAPE;
    const int64_t bytes = (int64_t)block_size * num_kv_heads * head_dim * elem_bytes(cache_dtype);
    if (bytes % 16 != 0 || bytes > ((int64_t)1 << 31)) return PKV_ERR_UNSUPPORTED;
    if (num_pairs == 0) return PKV_OK;
    if (!dst_k || !dst_v || !src_k || !src_v || !block_pairs) return PKV_ERR_NULL;
    if (!aligned16(dst_k) || !aligned16(dst_v) || !aligned16(src_k) || !aligned16(src_v) ||
        ((uintptr_t)block_pairs & 3u))
        return PKV_ERR_ALIGN;
    if ((src_k == dst_k) != (src_v == dst_v)) return PKV_ERR_SHAPE;
    CopyParams p;
    p.dk = dst_k;
    p.dv = dst_v;
    p.sk = src_k;
    p.sv = src_v;
    p.pairs = block_pairs;
    p.n = num_pairs;
    p.src_blocks = src_blocks;
    p.dst_blocks = dst_blocks;
    p.block_bytes = (uint32_t)bytes;
    return launch_status(launch_copy_blocks(p, stream));
}

int pkv_host_device_pointer(const void* host_ptr, void** device_ptr) {
    if (!host_ptr || !device_ptr) return PKV_ERR_NULL;
    *device_ptr = nullptr;
    void* d = nullptr;
    if (hipHostGetDevicePointer(&d, const_cast<void*>(host_ptr), 0) != hipSuccess || !d) {
        (void)hipGetLastError();           // leave no sticky error behind
        return PKV_ERR_HIP;
    }
    *device_ptr = d;
    return PKV_OK;
}

int pkv_paged_attention_decode_mixed(void* out, const void* query, pkv_dtype q_dtype,
                                     const void* k_cache, const void* v_cache,
                                     pkv_dtype cache_dtype, const int32_t* block_tables,
                                     int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                     const int32_t* seq_block_sizes, int32_t num_seqs,
                                     int32_t num_q_heads, int32_t num_kv_heads,
                                     int32_t head_dim, int32_t page_size, int32_t num_pages,
                                     int32_t max_seq_len, float scale, float k_scale,
                                     float v_scale, int32_t partition_size, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream) {
    if (!valid_dtype(q_dtype) || !valid_dtype(cache_dtype)) return PKV_ERR_DTYPE;
    if (!valid_decode_types(q_dtype, cache_dtype)) return PKV_ERR_DTYPE;
    const bool balanced = partition_size == PKV_PARTITION_BALANCED;
    if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        page_size <= 0 || num_pages <= 0 || max_blocks_per_seq <= 0 || max_seq_len <= 0 ||
        (partition_size < 0 && !balanced))
        return PKV_ERR_SHAPE;
    if (num_q_heads % num_kv_heads != 0) return PKV_ERR_SHAPE;
    if (num_kv_heads > 4096) return PKV_ERR_SHAPE;
    if (!(scale == scale) || !(k_scale == k_scale) || !(v_scale == v_scale)) return PKV_ERR_SHAPE;
    if (!supported_block_size(page_size)) return PKV_ERR_UNSUPPORTED;
    // the pool holds at least one block of the largest size; token counts
    // of whole tables (max_blocks_per_seq * 32) stay 32-bit on the device
    if ((int64_t)num_pages * page_size < 32) return PKV_ERR_SHAPE;
    if (max_blocks_per_seq > (1 << 25)) return PKV_ERR_SHAPE;
    if (partition_size > 0 && partition_size % 32 != 0) return PKV_ERR_SHAPE;
    const int G = num_q_heads / num_kv_heads;
    if (!decode_mfma_supported(q_dtype, cache_dtype, head_dim, G)) return PKV_ERR_UNSUPPORTED;
    if (!out || !query || !k_cache || !v_cache || !block_tables || !seq_lens ||
        !seq_block_sizes)
        return PKV_ERR_NULL;
    if (!aligned16(out) || !aligned16(query) || !aligned16(k_cache) || !aligned16(v_cache) ||
        ((uintptr_t)block_tables & 3u) || ((uintptr_t)seq_lens & 3u) ||
        ((uintptr_t)seq_block_sizes & 3u))
        return PKV_ERR_ALIGN;

    DecodeParams p;
    p.out = out;
    p.q = query;
    p.k = k_cache;
    p.v = v_cache;
    p.tables = block_tables;
    p.lens = seq_lens;
    p.ws_m = p.ws_l = p.ws_o = nullptr;
    p.ws_hdr = p.ws_pre = nullptr;
    p.nW = 0;
    p.epoch = 0;
    p.q_start = nullptr;
    p.max_groups = 0;
    p.col_blocks = 1;
    p.ws_len = nullptr;
    p.len_rows = 0;
    p.seq_bs = seq_block_sizes;
    p.page_shift = page_size == 8 ? 3 : (page_size == 16 ? 4 : 5);
    p.S = num_seqs;
    p.Hq = num_q_heads;
    p.Hkv = num_kv_heads;
    p.D = head_dim;
    p.G = G;
    p.bs = page_size;
    p.NB = num_pages;
    p.max_blocks = max_blocks_per_seq;
    const int64_t cap = (int64_t)max_blocks_per_seq * 32;
    p.len_cap = (int)(cap < max_seq_len ? cap : max_seq_len);
    p.P = partition_size;
    p.P_max = 1;
    const float ks = cache_dtype == PKV_FP8_E4M3 ? k_scale : 1.0f;
    p.scale_log2 = scale * ks * kLog2e;
    p.v_scale = cache_dtype == PKV_FP8_E4M3 ? v_scale : 1.0f;
    if (partition_size != 0) {
        WsLayout w;
        if (!ws_layout(num_seqs, num_q_heads, num_kv_heads, head_dim, max_seq_len,
                       partition_size, &w))
            return PKV_ERR_SHAPE;
        if (!workspace || workspace_bytes < w.bytes) return PKV_ERR_WORKSPACE;
        if (!aligned16(workspace)) return PKV_ERR_ALIGN;
        p.P_max = balanced ? 1 : w.P_max;
        p.ws_hdr = (int32_t*)workspace;
        p.ws_pre = (int32_t*)((char*)workspace + w.off_pre);
        p.ws_m = (float*)((char*)workspace + w.off_m);
        p.ws_l = (float*)((char*)workspace + w.off_l);
        p.ws_o = (float*)((char*)workspace + w.off_o);
    }
    if (balanced) {
        // the balanced split's walk over each sequence's own block size
        // (8-token tiles for 8-token blocks); pkv_paged_attention_reduce
        // merges the pieces as after a uniform pool
        const int64_t tiles = (int64_t)num_seqs * num_kv_heads * ((p.len_cap + 7) / 8);
        if (tiles > ((int64_t)1 << 31) - 1) return PKV_ERR_SHAPE;
        if (num_seqs > kBalancedMaxSeqs) return PKV_ERR_UNSUPPORTED;
        p.P = 0;
        p.nW = balanced_grid_waves(q_dtype, cache_dtype, head_dim, 16);
        p.epoch = next_call_number();
        return launch_status(launch_decode_balanced(q_dtype, cache_dtype, p, stream));
    }
    const int64_t units = (int64_t)num_seqs * p.P_max * num_kv_heads;
    if (units > ((int64_t)1 << 31) - 64) return PKV_ERR_SHAPE;
    return launch_status(launch_decode_mixed(q_dtype, cache_dtype, p, stream));
}

size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                  int32_t num_kv_heads, int32_t head_dim,
                                  int32_t max_seq_len, int32_t partition_size) {
    WsLayout w;
    if (!ws_layout(num_seqs, num_q_heads, num_kv_heads, head_dim, max_seq_len, partition_size,
                   &w))
        return 0;
    return w.bytes;
}

}  // extern "C"

namespace {

// Checks the arguments common to the decode entry points and fills the
// parameter block (everything but the workspace pieces).  Returns a
// negative status, with nothing enqueued, on a bad argument.
int prepare_decode(void* out, const void* query, int q_dtype, const void* k_cache,
                   const void* v_cache, int cache_dtype, const int32_t* block_tables,
                   int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t num_seqs,
                   int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                   int32_t block_size, int32_t num_blocks, int32_t max_seq_len, float scale,
                   float k_scale, float v_scale, int32_t partition_size, int32_t algo,
                   DecodeParams& p) {
    if (!valid_dtype(q_dtype) || !valid_dtype(cache_dtype)) return PKV_ERR_DTYPE;
    if (!valid_decode_types(q_dtype, cache_dtype)) return PKV_ERR_DTYPE;
    if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        block_size <= 0 || num_blocks <= 0 || max_blocks_per_seq <= 0 || max_seq_len <= 0 ||
        (partition_size < 0 && partition_size != PKV_PARTITION_BALANCED))
        return PKV_ERR_SHAPE;
    if (num_q_heads % num_kv_heads != 0) return PKV_ERR_SHAPE;
    if (num_kv_heads > 4096) return PKV_ERR_SHAPE;   // keeps in-block offsets 32-bit
    if (!(scale == scale) || !(k_scale == k_scale) || !(v_scale == v_scale)) return PKV_ERR_SHAPE;
    if (algo < PKV_ALGO_AUTO || algo > PKV_ALGO_MFMA) return PKV_ERR_UNSUPPORTED;
    if (!supported_block_size(block_size)) return PKV_ERR_UNSUPPORTED;
    if (partition_size > 0 && (partition_size % 16 != 0 || partition_size % block_size != 0))
        return PKV_ERR_SHAPE;
    if (!out || !query || !k_cache || !v_cache || !block_tables || !seq_lens)
        return PKV_ERR_NULL;
    if (!aligned16(out) || !aligned16(query) || !aligned16(k_cache) || !aligned16(v_cache) ||
        ((uintptr_t)block_tables & 3u) || ((uintptr_t)seq_lens & 3u))
        return PKV_ERR_ALIGN;

    p.out = out;
    p.q = query;
    p.k = k_cache;
    p.v = v_cache;
    p.tables = block_tables;
    p.lens = seq_lens;
    p.ws_m = p.ws_l = p.ws_o = nullptr;
    p.ws_hdr = p.ws_pre = nullptr;
    p.nW = 0;
    p.epoch = 0;
    p.q_start = nullptr;
    p.max_groups = 0;
    p.col_blocks = 1;
    p.ws_len = nullptr;
    p.len_rows = 0;
    p.seq_bs = nullptr;
    p.page_shift = 0;
    p.S = num_seqs;
    p.Hq = num_q_heads;
    p.Hkv = num_kv_heads;
    p.D = head_dim;
    p.G = num_q_heads / num_kv_heads;
    p.bs = block_size;
    p.NB = num_blocks;
    p.max_blocks = max_blocks_per_seq;
    const int64_t cap = (int64_t)max_blocks_per_seq * block_size;
    p.len_cap = (int)(cap < max_seq_len ? cap : max_seq_len);
    p.P = partition_size;
    p.P_max = 1;
    const float ks = cache_dtype == PKV_FP8_E4M3 ? k_scale : 1.0f;
    p.scale_log2 = scale * ks * kLog2e;
    p.v_scale = cache_dtype == PKV_FP8_E4M3 ? v_scale : 1.0f;
    return PKV_OK;
}

// The balanced split's own limits: matrix-core types, the batch held in
// LDS, tile counts 32-bit on the device.
int balanced_supported(int q_dtype, int cache_dtype, const DecodeParams& p) {
    const int64_t tiles = (int64_t)p.S * p.Hkv * ((p.len_cap + 15) / 16);
    if (tiles > ((int64_t)1 << 31) - 1) return PKV_ERR_SHAPE;
    if (!decode_mfma_supported(q_dtype, cache_dtype, p.D, p.G) || p.S > kBalancedMaxSeqs)
        return PKV_ERR_UNSUPPORTED;
    return PKV_OK;
}

// ---- the decode call that allocates nothing --------------------------------
//
// Its workspace is `scratch`, one file-scope device array of kScratchBytes.
// HIP gives each GPU that loads the library its own copy at its own
// address, held until the process ends.  In host code the array's name is
// only a stand-in for the symbol: the device address of a GPU's copy comes
// from hipGetSymbolAddress, asked once per device with that device current
// and kept in g_scratch, and only that address is ever handed to a kernel.
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) char scratch[kScratchBytes];
std::atomic<char*> g_scratch[kMaxDevices];

// This device's copy of `scratch` (nullptr if HIP cannot give it).
char* scratch_on(int dev) {
    char* ptr = g_scratch[dev].load(std::memory_order_acquire);
    if (ptr) return ptr;
    void* d = nullptr;
    if (hipGetSymbolAddress(&d, HIP_SYMBOL(scratch)) != hipSuccess || !d) {
        (void)hipGetLastError();           // leave no sticky error behind
        return nullptr;
    }
    g_scratch[dev].store((char*)d, std::memory_order_release);
    return (char*)d;
}

// The balanced workspace sized for a grid of nW wavefronts (entries for
// the chunk bound of that grid rather than of the largest one).
inline size_t balanced_bytes_for_grid(int S, int Hkv, int G, int D, int nW, WsLayout* w) {
    const size_t n = (size_t)2 * (size_t)max_chunks(nW) * (size_t)G;
    w->P_max = 0;
    w->off_pre = 256;
    w->off_m = round_up(w->off_pre + 4 * ((size_t)S + 1) + 8 * (size_t)S * (size_t)Hkv, 256);
    w->off_l = w->off_m + round_up(n * 4, 256);
    w->off_o = w->off_l + round_up(n * 4, 256);
    w->bytes = w->off_o + n * (size_t)D * 4;
    return w->bytes;
}

}  // namespace

extern "C" {

int pkv_paged_attention_decode(void* out, const void* query, pkv_dtype q_dtype,
                               const void* k_cache, const void* v_cache,
                               pkv_dtype cache_dtype, const int32_t* block_tables,
                               int32_t max_blocks_per_seq, const int32_t* seq_lens,
                               int32_t num_seqs, int32_t num_q_heads,
                               int32_t num_kv_heads, int32_t head_dim,
                               int32_t block_size, int32_t num_blocks,
                               int32_t max_seq_len, float scale, float k_scale,
                               float v_scale, int32_t partition_size,
                               void* workspace, size_t workspace_bytes,
                               int32_t algo, hipStream_t stream) {
    DecodeParams p;
    const int rc = prepare_decode(out, query, q_dtype, k_cache, v_cache, cache_dtype,
                                  block_tables, max_blocks_per_seq, seq_lens, num_seqs,
                                  num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                                  max_seq_len, scale, k_scale, v_scale, partition_size, algo, p);
    if (rc != PKV_OK) return rc;
    const bool balanced = partition_size == PKV_PARTITION_BALANCED;
    if (partition_size != 0) {
        WsLayout w;
        if (!ws_layout(num_seqs, num_q_heads, num_kv_heads, head_dim, max_seq_len,
                       partition_size, &w))
            return PKV_ERR_SHAPE;
        if (!workspace) return PKV_ERR_WORKSPACE;
        if (workspace_bytes < w.bytes) return PKV_ERR_WORKSPACE;
        if (!aligned16(workspace)) return PKV_ERR_ALIGN;
        p.P_max = balanced ? 1 : w.P_max;
        p.ws_hdr = (int32_t*)workspace;
        p.ws_pre = (int32_t*)((char*)workspace + w.off_pre);
        p.ws_m = (float*)((char*)workspace + w.off_m);
        p.ws_l = (float*)((char*)workspace + w.off_l);
        p.ws_o = (float*)((char*)workspace + w.off_o);
    }
    const int64_t units = (int64_t)num_seqs * p.P_max * num_kv_heads;
    if (units > ((int64_t)1 << 31) - 64) return PKV_ERR_SHAPE;

    const bool mfma_ok = decode_mfma_supported(q_dtype, cache_dtype, head_dim, p.G);
    const bool valu_ok = decode_valu_supported(q_dtype, cache_dtype, head_dim, p.G);
    if (balanced) {
        const int bal = balanced_supported(q_dtype, cache_dtype, p);
        if (bal != PKV_OK) return bal;
        if (algo == PKV_ALGO_VALU) return PKV_ERR_UNSUPPORTED;
        p.P = 0;
        p.nW = balanced_grid_waves(q_dtype, cache_dtype, head_dim, block_size);
        p.epoch = next_call_number();
        return launch_status(launch_decode_balanced(q_dtype, cache_dtype, p, stream));
    }
    if (algo == PKV_ALGO_MFMA || (algo == PKV_ALGO_AUTO && mfma_ok)) {
        if (!mfma_ok) return PKV_ERR_UNSUPPORTED;
        return launch_status(launch_decode_mfma(q_dtype, cache_dtype, p, stream));
    }
    if (!valu_ok) return PKV_ERR_UNSUPPORTED;
    return launch_status(launch_decode_valu(q_dtype, cache_dtype, p, stream));
}

int pkv_paged_attention_reduce(void* out, pkv_dtype out_dtype, const void* workspace,
                               size_t workspace_bytes, const int32_t* seq_lens,
                               int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                               int32_t head_dim, int32_t max_seq_len, int32_t partition_size,
                               hipStream_t stream) {
    if (!valid_dtype(out_dtype) || out_dtype == PKV_FP8_E4M3) return PKV_ERR_DTYPE;
    const bool balanced = partition_size == PKV_PARTITION_BALANCED;
    if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        max_seq_len <= 0 || (partition_size <= 0 && !balanced))
        return PKV_ERR_SHAPE;
    if (num_q_heads % num_kv_heads != 0) return PKV_ERR_SHAPE;
    if (!balanced && partition_size % 16 != 0) return PKV_ERR_SHAPE;
    if (head_dim != 64 && head_dim != 128) return PKV_ERR_UNSUPPORTED;
    if (balanced && num_seqs > kBalancedMaxSeqs) return PKV_ERR_UNSUPPORTED;
    WsLayout w;
    if (!ws_layout(num_seqs, num_q_heads, num_kv_heads, head_dim, max_seq_len, partition_size,
                   &w))
        return PKV_ERR_SHAPE;
    if (!out || !seq_lens) return PKV_ERR_NULL;
    if (!workspace || workspace_bytes < w.bytes) return PKV_ERR_WORKSPACE;
    if (!aligned16(out) || !aligned16(workspace) || ((uintptr_t)seq_lens & 3u))
        return PKV_ERR_ALIGN;
    if ((int64_t)num_seqs * num_q_heads > ((int64_t)1 << 31) - 64) return PKV_ERR_SHAPE;
    ReduceParams p;
    p.out = out;
    p.ws_hdr = (const int32_t*)workspace;
    p.ws_pre = (const int32_t*)((const char*)workspace + w.off_pre);
    p.ws_m = (const float*)((const char*)workspace + w.off_m);
    p.ws_l = (const float*)((const char*)workspace + w.off_l);
    p.ws_o = (const float*)((const char*)workspace + w.off_o);
    p.lens = seq_lens;
    p.S = num_seqs;
    p.Hq = num_q_heads;
    p.Hkv = num_kv_heads;
    p.D = head_dim;
    p.P = balanced ? 0 : partition_size;
    p.P_max = w.P_max;
    p.len_cap = max_seq_len;
    p.q_start = nullptr;
    p.S_seq = num_seqs;
    set_group(p);
    if (balanced) return launch_status(launch_reduce_balanced(out_dtype, p, stream));
    return launch_status(launch_reduce(out_dtype, p, stream));
}

int pkv_paged_attention_decode_noalloc(void* out, const void* query, pkv_dtype q_dtype,
                                       const void* k_cache, const void* v_cache,
                                       pkv_dtype cache_dtype, const int32_t* block_tables,
                                       int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                       int32_t num_seqs, int32_t num_q_heads,
                                       int32_t num_kv_heads, int32_t head_dim,
                                       int32_t block_size, int32_t num_blocks,
                                       int32_t max_seq_len, float scale, float k_scale,
                                       float v_scale, hipStream_t stream) {
    DecodeParams p;
    int rc = prepare_decode(out, query, q_dtype, k_cache, v_cache, cache_dtype, block_tables,
                            max_blocks_per_seq, seq_lens, num_seqs, num_q_heads, num_kv_heads,
                            head_dim, block_size, num_blocks, max_seq_len, scale, k_scale,
                            v_scale, PKV_PARTITION_BALANCED, PKV_ALGO_MFMA, p);
    if (rc != PKV_OK) return rc;
    rc = balanced_supported(q_dtype, cache_dtype, p);
    if (rc != PKV_OK) return rc;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PKV_ERR_HIP;
    p.P = 0;
    p.P_max = 1;
    p.nW = balanced_grid_waves(q_dtype, cache_dtype, head_dim, block_size);
    WsLayout w;
    if (balanced_bytes_for_grid(num_seqs, num_kv_heads, p.G, head_dim, p.nW, &w) > kScratchBytes)
        return PKV_ERR_SCRATCH;
    char* ws = scratch_on(dev);
    if (!ws) return PKV_ERR_HIP;
    p.ws_hdr = (int32_t*)ws;
    p.ws_pre = (int32_t*)(ws + w.off_pre);
    p.ws_m = (float*)(ws + w.off_m);
    p.ws_l = (float*)(ws + w.off_l);
    p.ws_o = (float*)(ws + w.off_o);
    p.epoch = next_call_number();
    hipError_t e = launch_decode_balanced(q_dtype, cache_dtype, p, stream);
    if (e != hipSuccess) return launch_status(e);
    // the reduce of the same split, on the same pieces of the array
    ReduceParams r;
    r.out = out;
    r.ws_hdr = p.ws_hdr;
    r.ws_pre = p.ws_pre;
    r.ws_m = p.ws_m;
    r.ws_l = p.ws_l;
    r.ws_o = p.ws_o;
    r.lens = seq_lens;
    r.S = num_seqs;
    r.Hq = num_q_heads;
    r.Hkv = num_kv_heads;
    r.D = head_dim;
    r.P = 0;
    r.P_max = 0;
    r.len_cap = max_seq_len;
    r.q_start = nullptr;
    r.S_seq = num_seqs;
    set_group(r);
    return launch_status(launch_reduce_balanced(q_dtype, r, stream));
}

}  // extern "C"
