// C ABI of libcsa2: argument validation, workspace carving and launch order.
// Every entry point validates on the host, then enqueues kernels on the
// caller's stream and returns; nothing here synchronises with the device.
#include <cmath>
#include <cstring>
#include <mutex>

#include "csa2_internal.h"

using namespace csa2;

namespace {

thread_local int32_t g_last_hip_error = 0;

csa2_status hip_fail(hipError_t e) {
    g_last_hip_error = (int32_t)e;
    return CSA2_ERR_HIP;
}

size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

// Validates the batch descriptor and derives the launch geometry.
csa2_status batch_geometry(const csa2_batch* b, Geometry* g) {
    if (!b || b->n_seq < 1 || b->total_q < 1 || b->ratio < 1) return CSA2_ERR_INVALID_ARG;
    if (!b->h_entry_off || !b->h_q_off || !b->h_q_pos || !b->d_entry_off || !b->d_q_off || !b->d_q_pos ||
        !b->d_row_seq)
        return CSA2_ERR_INVALID_ARG;
    if (b->h_entry_off[0] != 0 || b->h_q_off[0] != 0 || b->h_q_off[b->n_seq] != b->total_q) return CSA2_ERR_INVALID_ARG;
    int64_t max_n = 0;
    int max_q = 0;
    for (int s = 0; s < b->n_seq; ++s) {
        const int64_t n = b->h_entry_off[s + 1] - b->h_entry_off[s];
        const int nq = b->h_q_off[s + 1] - b->h_q_off[s];
        if (n < 0 || nq < 0) return CSA2_ERR_INVALID_ARG;
        if (n > max_n) max_n = n;
        if (nq > max_q) max_q = nq;
    }
    if (max_n >= ((int64_t)1 << 31)) return CSA2_ERR_UNSUPPORTED;
    for (int r = 0; r < b->total_q; ++r)
        if (b->h_q_pos[r] < 0) return CSA2_ERR_INVALID_ARG;
    g->n_seq = b->n_seq;
    g->total_q = b->total_q;
    g->ratio = b->ratio;
    g->max_entries = max_n;
    g->max_q_per_seq = max_q;
    return CSA2_OK;
}

csa2_status check_ws(void* ws, size_t ws_bytes, size_t need) {
    if (need == 0) return CSA2_OK;
    if (!ws || ws_bytes < need || ((uintptr_t)ws & 255)) return CSA2_ERR_WORKSPACE;
    return CSA2_OK;
}

csa2_status check_swa(const csa2_batch* b, const csa2_swa_layout* sw) {
    if (!sw || sw->window < 1 || sw->window > 1024) return sw && sw->window > 1024 ? CSA2_ERR_UNSUPPORTED : CSA2_ERR_INVALID_ARG;
    if (sw->fmt != CSA2_SWA_BF16 && sw->fmt != CSA2_SWA_MXFP8) return CSA2_ERR_UNSUPPORTED;
    if (!sw->h_row_off || !sw->h_pos0 || !sw->h_len || !sw->d_row_off || !sw->d_pos0) return CSA2_ERR_INVALID_ARG;
    if ((sw->h_replay_s == nullptr) != (sw->d_replay_s == nullptr)) return CSA2_ERR_INVALID_ARG;
    for (int s = 0; s < b->n_seq; ++s) {
        if (sw->h_len[s] < 0 || sw->h_pos0[s] < 0 || sw->h_row_off[s] < 0) return CSA2_ERR_INVALID_ARG;
        const int64_t rep = sw->h_replay_s ? sw->h_replay_s[s] : 0;
        for (int r = b->h_q_off[s]; r < b->h_q_off[s + 1]; ++r) {
            const int64_t t = b->h_q_pos[r];
            int64_t lo = t - sw->window + 1;
            if (lo < rep) lo = rep;
            if (lo > t) continue;  // empty window
            if (lo < sw->h_pos0[s] || t >= (int64_t)sw->h_pos0[s] + sw->h_len[s]) return CSA2_ERR_INVALID_ARG;
        }
    }
    return CSA2_OK;
}

size_t pool_ws_bytes(const Geometry& g, int block) {
    const int64_t nb = (g.max_entries + block - 1) / block;
    return al256((size_t)g.total_q * (size_t)(nb > 0 ? nb : 1) * 4) + topk_ws_bytes(g.total_q);
}

struct ChainWs {
    size_t scores, pool_scores, pool_ws, idx_cur, idx_empty, pool_out, tiles, attn, attn_bytes, total;
    int64_t tstride;  // tile maxima per row
};

ChainWs chain_ws(const Geometry& g, int K, int block, int max_blocks) {
    ChainWs w{};
    size_t off = 0;
    w.scores = off;  // score rows, or the scan's per-chunk lists and counts (never both in one layer)
    const size_t rows_bytes = al256((size_t)g.total_q * (size_t)(g.max_entries > 0 ? g.max_entries : 1) * 4);
    const size_t lists_bytes = al256(local_lists_bytes(g)) + 2 * al256(local_counts_bytes(g));  // lists, counts, bounds
    off += rows_bytes > lists_bytes ? rows_bytes : lists_bytes;
    w.pool_scores = off;
    off += al256((size_t)g.total_q * (size_t)max_blocks * block * 4);
    w.pool_ws = off;  // block scores + Top-K workspace (the Top-K calls reuse its tail)
    off += pool_ws_bytes(g, block);
    w.idx_cur = off;
    off += al256((size_t)g.total_q * K * 4);
    w.idx_empty = off;
    off += al256((size_t)g.total_q * K * 4);
    w.pool_out = off;
    off += al256((size_t)g.total_q * max_blocks * 4) + al256((size_t)g.total_q * max_blocks * block * 4) +
           al256((size_t)g.total_q * 4);
    w.tiles = off;  // the prefill scorer's tile maxima [total_q][tstride], then one tile bound per row
    w.tstride = (g.max_entries + kTile - 1) / kTile;
    if (w.tstride < 1) w.tstride = 1;
    off += al256((size_t)g.total_q * (size_t)w.tstride * 4) + al256((size_t)g.total_q * 4);
    w.attn = off;  // attention partials for 64 heads and a 128-row window
    w.attn_bytes = attn_ws_bytes(g, 64, attn_splits(g, 64, K, 128));
    off += al256(w.attn_bytes);
    w.total = off;
    return w;
}

// The index scan of a Full layer, between the caller's events the first time.
hipError_t timed_scan(const ScoreLaunch& sa, const csa2_chain_params* p, bool* timed, hipStream_t stream) {
    // the events are stamped by the kernel's own dispatch (no extra packets
    // in the queue around it)
    const bool rec = !*timed && (p->scan_begin || p->scan_end);
    ScoreLaunch a = sa;
    if (rec) {
        a.ev_begin = p->scan_begin;
        a.ev_end = p->scan_end;
    }
    const hipError_t e = launch_index_score(a, stream);
    if (e != hipSuccess) return e;
    *timed = true;
    return hipSuccess;
}

__global__ void k_fill_i32(int32_t* p, int64_t n, int32_t v) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = v;
}

// Scratch of csa2_topk_noalloc: the Top-K workspace of up to kNoAllocTopkRows
// query rows, a file-scope device array that each GPU the library runs on
// holds until the process ends.  Host code never passes `scratch` itself to a
// kernel (in host code the name is a stand-in, not the device address): the
// address comes from hipGetSymbolAddress, once per device, with that device
// current.
constexpr int kNoAllocTopkRows = 256;
constexpr size_t kNoAllocScratchBytes =
    ((size_t)kNoAllocTopkRows * kHistBins * 4 + 255) / 256 * 256 +
    ((size_t)kNoAllocTopkRows * sizeof(RowSel) + 255) / 256 * 256 +
    ((size_t)kNoAllocTopkRows * kCandCap * 8 + 255) / 256 * 256;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on `dev` (nullptr on failure; *err holds
// the HIP error).
void* scratch_on(int dev, hipError_t* err) {
    *err = hipSuccess;
    if (dev < 0 || dev >= kMaxDevices) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev]) return g_scratch_ptr[dev];
    int cur = 0;
    if ((*err = hipGetDevice(&cur)) != hipSuccess) return nullptr;
    if (cur != dev && (*err = hipSetDevice(dev)) != hipSuccess) return nullptr;
    void* ptr = nullptr;
    *err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != dev) {
        const hipError_t e2 = hipSetDevice(cur);
        if (*err == hipSuccess) *err = e2;
    }
    if (*err != hipSuccess || !ptr) {
        if (*err == hipSuccess) *err = hipErrorInvalidSymbol;
        return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
    return ptr;
}

}  // namespace

extern "C" {

CSA2_API int32_t csa2_version(void) { return 1; }

CSA2_API int32_t csa2_last_hip_error(void) { return g_last_hip_error; }

CSA2_API const char* csa2_status_string(csa2_status s) {
    switch (s) {
        case CSA2_OK: return "ok";
        case CSA2_ERR_INVALID_ARG: return "invalid argument";
        case CSA2_ERR_UNSUPPORTED: return "unsupported size or format";
        case CSA2_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
        case CSA2_ERR_HIP: return "HIP launch error";
        case CSA2_ERR_SCRATCH: return "the problem exceeds the static scratch of the allocation-free call";
        default: return "unknown status";
    }
}

CSA2_API size_t csa2_workspace_size(int32_t which, const csa2_batch* batch, int32_t K, int32_t max_blocks,
                                    int32_t n_layers) {
    Geometry g;
    if (batch_geometry(batch, &g) != CSA2_OK) return 0;
    switch (which) {
        case CSA2_WS_TOPK: return topk_ws_bytes(g.total_q);
        case CSA2_WS_BLOCK_POOL: return pool_ws_bytes(g, 8);
        case CSA2_WS_SPARSE_ATTN:  // for 64 heads and a 128-row window; a smaller workspace means fewer splits
            if (K < 1) return 0;
            return attn_ws_bytes(g, 64, attn_splits(g, 64, K, 128));
        case CSA2_WS_LAYER_CHAIN:
            if (K < 1 || max_blocks < 1 || n_layers < 1) return 0;
            return chain_ws(g, K, 8, max_blocks).total;
        default: return 0;
    }
}

CSA2_API csa2_status csa2_index_score(const csa2_batch* batch, int32_t H, int32_t q_fmt, const void* q,
                                      const uint8_t* q_sc, const float* w, const uint8_t* k_fp4,
                                      const uint8_t* k_sc, const int32_t* cand, int32_t cand_stride,
                                      float* scores, int64_t score_stride, uint32_t* hist, hipStream_t stream) {
    Geometry g;
    csa2_status st = batch_geometry(batch, &g);
    if (st) return st;
    if (!q || !q_sc || !w || !k_fp4 || !k_sc || !scores) return CSA2_ERR_INVALID_ARG;
    if (q_fmt != CSA2_Q_FP4 && q_fmt != CSA2_Q_FP8 && q_fmt != CSA2_Q_MXFP4) return CSA2_ERR_INVALID_ARG;
    if (H != 32 && H != 64) return CSA2_ERR_UNSUPPORTED;
    if (cand) {
        if (q_fmt == CSA2_Q_FP8) return CSA2_ERR_UNSUPPORTED;
        if (cand_stride < 1 || score_stride < cand_stride) return CSA2_ERR_INVALID_ARG;
    } else if (score_stride < g.max_entries || score_stride < 1) {
        return CSA2_ERR_INVALID_ARG;
    }
    if (hist && (q_fmt == CSA2_Q_FP8 || (!cand && g.max_q_per_seq > 4))) return CSA2_ERR_UNSUPPORTED;
    ScoreLaunch a{batch, g, H, q_fmt, (const uint8_t*)q, q_sc, w, k_fp4, k_sc, cand, cand_stride, scores, score_stride,
                  hist};
    hipError_t e = launch_index_score(a, stream);
    return e == hipSuccess ? CSA2_OK : hip_fail(e);
}

CSA2_API csa2_status csa2_rope_cast(int64_t n_rows, int32_t heads, const float* in, const float* rope_cs,
                                    int32_t inverse, uint16_t* out_bf16, hipStream_t stream) {
    if (n_rows < 0 || heads < 1) return CSA2_ERR_INVALID_ARG;
    if (n_rows == 0) return CSA2_OK;
    if (!in || !rope_cs || !out_bf16) return CSA2_ERR_INVALID_ARG;
    if (((uintptr_t)in | (uintptr_t)rope_cs | (uintptr_t)out_bf16) & 15) return CSA2_ERR_INVALID_ARG;
    if (n_rows > INT64_MAX / heads || (n_rows * heads + 3) / 4 > 0x7FFFFFFF) return CSA2_ERR_UNSUPPORTED;
    const hipError_t e = launch_rope_cast(n_rows, heads, in, rope_cs, inverse ? 1 : 0, out_bf16, stream);
    return e == hipSuccess ? CSA2_OK : hip_fail(e);
}

CSA2_API csa2_status csa2_index_k_project(int64_t n, const float* x, const float* rope_cs, const float* W,
                                          const int64_t* dst_row, int64_t n_rows, int32_t q_fmt, uint8_t* k_fp4,
                                          uint8_t* k_sc, hipStream_t stream) {
    if (n < 0) return CSA2_ERR_INVALID_ARG;
    if (q_fmt != CSA2_Q_FP4 && q_fmt != CSA2_Q_FP8 && q_fmt != CSA2_Q_MXFP4) return CSA2_ERR_INVALID_ARG;
    if (n == 0) return CSA2_OK;
    if (!x || !W || !dst_row || !k_fp4 || !k_sc || n_rows < 1) return CSA2_ERR_INVALID_ARG;
    if (((uintptr_t)x | (uintptr_t)rope_cs | (uintptr_t)W | (uintptr_t)k_fp4) & 15) return CSA2_ERR_INVALID_ARG;
    if ((n + 63) / 64 > 0x7FFFFFFF) return CSA2_ERR_UNSUPPORTED;
    const hipError_t e =
        launch_index_k_project(n, x, rope_cs, W, dst_row, n_rows, q_fmt == CSA2_Q_MXFP4, k_fp4, k_sc, stream);
    return e == hipSuccess ? CSA2_OK : hip_fail(e);
}

CSA2_API csa2_status csa2_compress(int64_t n_entries, int32_t m, const float* c_tok, const float* z_tok, float* out,
                                   hipStream_t stream) {
    if (n_entries < 0) return CSA2_ERR_INVALID_ARG;
    if (m < 1 || m > 16) return CSA2_ERR_UNSUPPORTED;
    if (n_entries == 0) return CSA2_OK;
    if (!c_tok || !z_tok || !out) return CSA2_ERR_INVALID_ARG;
    if (((uintptr_t)c_tok | (uintptr_t)z_tok | (uintptr_t)out) & 15) return CSA2_ERR_INVALID_ARG;
    if ((n_entries + 1) / 2 > 0x7FFFFFFF) return CSA2_ERR_UNSUPPORTED;
    const hipError_t e = launch_compress(n_entries, m, c_tok, z_tok, out, stream);
    return e == hipSuccess ? CSA2_OK : hip_fail(e);
}

CSA2_API csa2_status csa2_kv_append(int64_t n, const float* x, const float* rope_cs, const int64_t* dst_row,
                                    int64_t n_rows, int32_t kv_fmt, uint8_t* kv_fp4, uint8_t* kv_sc,
                                    hipStream_t stream) {
    if (n < 0) return CSA2_ERR_INVALID_ARG;
    if (kv_fmt != CSA2_KV_MXFP4 && kv_fmt != CSA2_KV_E4M3_16) return CSA2_ERR_UNSUPPORTED;
    if (n == 0) return CSA2_OK;
    if (!x || !rope_cs || !dst_row || !kv_fp4 || !kv_sc || n_rows < 1) return CSA2_ERR_INVALID_ARG;
    if ((n + 3) / 4 > 0x7FFFFFFF) return CSA2_ERR_UNSUPPORTED;
    if (((uintptr_t)x | (uintptr_t)rope_cs | (uintptr_t)kv_fp4) & 15) return CSA2_ERR_INVALID_ARG;
    const hipError_t e = launch_kv_append(n, x, rope_cs, dst_row, n_rows, kv_fmt, kv_fp4, kv_sc, stream);
    return e == hipSuccess ? CSA2_OK : hip_fail(e);
}

}  // extern "C"

namespace {

// Host validation shared by csa2_topk and csa2_topk_noalloc.
csa2_status topk_args(const csa2_batch* batch, const float* scores, int64_t score_stride, const int32_t* cand,
                      int32_t cand_stride, const int32_t* cand_count, int32_t K, int32_t* idx, Geometry* g,
                      int64_t* max_slots) {
    csa2_status st = batch_geometry(batch, g);
    if (st) return st;
    if (!scores || !idx) return CSA2_ERR_INVALID_ARG;
    if (K < 1 || K > kMaxK) return K < 1 ? CSA2_ERR_INVALID_ARG : CSA2_ERR_UNSUPPORTED;
    *max_slots = g->max_entries;
    if (cand) {
        if (!cand_count || cand_stride < 1 || score_stride < cand_stride) return CSA2_ERR_INVALID_ARG;
        *max_slots = cand_stride;
    } else if (score_stride < g->max_entries) {
        return CSA2_ERR_INVALID_ARG;
    }
    return CSA2_OK;
}

}  // namespace

extern "C" {

CSA2_API csa2_status csa2_topk(const csa2_batch* batch, const float* scores, int64_t score_stride,
                               const int32_t* cand, int32_t cand_stride, const int32_t* cand_count, int32_t K,
                               const uint32_t* hist, int32_t* idx, void* ws, size_t ws_bytes, hipStream_t stream) {
    Geometry g;
    int64_t max_slots = 0;
    csa2_status st = topk_args(batch, scores, score_stride, cand, cand_stride, cand_count, K, idx, &g, &max_slots);
    if (st) return st;
    if ((st = check_ws(ws, ws_bytes, topk_ws_bytes(g.total_q)))) return st;
    TopkLaunch a{};
    a.b = batch;
    a.g = g;
    a.scores = scores;
    a.stride = score_stride;
    a.max_slots = max_slots;
    a.cand = cand;
    a.cand_stride = cand_stride;
    a.cand_count = cand_count;
    a.block_mode = 0;
    a.block = 1;
    a.K = K;
    a.idx = idx;
    a.ws = ws;
    a.hist = hist;
    hipError_t e = launch_topk(a, stream);
    return e == hipSuccess ? CSA2_OK : hip_fail(e);
}

CSA2_API csa2_status csa2_topk_noalloc(const csa2_batch* batch, const float* scores, int64_t score_stride,
                                       const int32_t* cand, int32_t cand_stride, const int32_t* cand_count, int32_t K,
                                       const uint32_t* hist, int32_t* idx, hipStream_t stream) {
    Geometry g;
    int64_t max_slots = 0;
    csa2_status st = topk_args(batch, scores, score_stride, cand, cand_stride, cand_count, K, idx, &g, &max_slots);
    if (st) return st;
    if (topk_ws_bytes(g.total_q) > kNoAllocScratchBytes) return CSA2_ERR_SCRATCH;
    int dev = 0;
    hipError_t e = hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess) return hip_fail(e);
    void* ws = scratch_on(dev, &e);
    if (!ws) return hip_fail(e);
    return csa2_topk(batch, scores, score_stride, cand, cand_stride, cand_count, K, hist, idx, ws,
                     kNoAllocScratchBytes, stream);
}

CSA2_API csa2_status csa2_block_pool(const csa2_batch* batch, const float* scores, int64_t score_stride,
                                     int32_t block, int32_t max_blocks, int32_t* blocks, int32_t* pool_pos,
                                     int32_t* pool_count, void* ws, size_t ws_bytes, hipStream_t stream) {
    Geometry g;
    csa2_status st = batch_geometry(batch, &g);
    if (st) return st;
    if (!scores || !blocks || !pool_pos || !pool_count) return CSA2_ERR_INVALID_ARG;
    if (block != 8) return block < 1 ? CSA2_ERR_INVALID_ARG : CSA2_ERR_UNSUPPORTED;
    if (max_blocks < 1 || max_blocks > kMaxK) return max_blocks < 1 ? CSA2_ERR_INVALID_ARG : CSA2_ERR_UNSUPPORTED;
    if (score_stride < g.max_entries) return CSA2_ERR_INVALID_ARG;
    if ((st = check_ws(ws, ws_bytes, pool_ws_bytes(g, block)))) return st;
    const int64_t nb = (g.max_entries + block - 1) / block;
    PoolLaunch a{};
    a.b = batch;
    a.g = g;
    a.scores = scores;
    a.stride = score_stride;
    a.block = block;
    a.max_blocks = max_blocks;
    a.blocks = blocks;
    a.pool_pos = pool_pos;
    a.pool_count = pool_count;
    a.bscores = (float*)ws;
    a.bstride = nb > 0 ? nb : 1;
    a.topk_ws = (char*)ws + al256((size_t)g.total_q * (size_t)a.bstride * 4);
    hipError_t e = launch_block_pool(a, stream);
    return e == hipSuccess ? CSA2_OK : hip_fail(e);
}

CSA2_API csa2_status csa2_gather_dequant(const csa2_batch* batch, int32_t kv_fmt, const uint8_t* kv_fp4,
                                         const uint8_t* kv_sc, const int32_t* idx, int32_t K, uint16_t* out_bf16,
                                         hipStream_t stream) {
    Geometry g;
    csa2_status st = batch_geometry(batch, &g);
    if (st) return st;
    if (kv_fmt != CSA2_KV_MXFP4 && kv_fmt != CSA2_KV_E4M3_16) return CSA2_ERR_UNSUPPORTED;
    if (!kv_fp4 || !kv_sc || !idx || !out_bf16) return CSA2_ERR_INVALID_ARG;
    if (K < 1 || K > 4096) return K < 1 ? CSA2_ERR_INVALID_ARG : CSA2_ERR_UNSUPPORTED;
    hipError_t e = launch_gather_dequant(batch, g, kv_fmt, kv_fp4, kv_sc, idx, K, out_bf16, stream);
    return e == hipSuccess ? CSA2_OK : hip_fail(e);
}

CSA2_API csa2_status csa2_sparse_attn(const csa2_batch* batch, int32_t Hm, const uint16_t* q_bf16, int32_t kv_fmt,
                                      const uint8_t* kv_fp4, const uint8_t* kv_sc, const int32_t* idx, int32_t K,
                                      const void* swa_rows, const csa2_swa_layout* swa, float softmax_scale,
                                      float* out, float* lse, void* ws, size_t ws_bytes, hipStream_t stream) {
    Geometry g;
    csa2_status st = batch_geometry(batch, &g);
    if (st) return st;
    if (!q_bf16 || !kv_fp4 || !kv_sc || !idx || !swa_rows || !out) return CSA2_ERR_INVALID_ARG;
    if (kv_fmt != CSA2_KV_MXFP4 && kv_fmt != CSA2_KV_E4M3_16) return CSA2_ERR_UNSUPPORTED;
    if (Hm < 16 || Hm % 16) return Hm < 1 ? CSA2_ERR_INVALID_ARG : CSA2_ERR_UNSUPPORTED;
    if (K < 1 || K > kMaxK) return K < 1 ? CSA2_ERR_INVALID_ARG : CSA2_ERR_UNSUPPORTED;
    if (!(softmax_scale > 0.0f) || !std::isfinite(softmax_scale)) return CSA2_ERR_INVALID_ARG;
    if ((st = check_swa(batch, swa))) return st;
    if (ws && ((uintptr_t)ws & 255)) return CSA2_ERR_WORKSPACE;
    AttnLaunch a{batch, g, Hm, q_bf16, kv_fp4, kv_sc, idx, K, swa_rows, swa, softmax_scale, out, lse, ws,
                 ws ? ws_bytes : 0, kv_fmt};
    hipError_t e = launch_sparse_attn(a, stream);
    return e == hipSuccess ? CSA2_OK : hip_fail(e);
}

CSA2_API csa2_status csa2_sparse_attn_rope(const csa2_batch* batch, int32_t Hm, const uint16_t* q_bf16,
                                           const float* rope_cs, int32_t kv_fmt, const uint8_t* kv_fp4,
                                           const uint8_t* kv_sc, const int32_t* idx, int32_t K, const void* swa_rows,
                                           const csa2_swa_layout* swa, float softmax_scale, uint16_t* out_bf16,
                                           float* lse, void* ws, size_t ws_bytes, hipStream_t stream) {
    Geometry g;
    csa2_status st = batch_geometry(batch, &g);
    if (st) return st;
    if (!q_bf16 || !rope_cs || !kv_fp4 || !kv_sc || !idx || !swa_rows || !out_bf16) return CSA2_ERR_INVALID_ARG;
    if (((uintptr_t)q_bf16 | (uintptr_t)rope_cs) & 15 || ((uintptr_t)out_bf16 & 3)) return CSA2_ERR_INVALID_ARG;
    if (kv_fmt != CSA2_KV_MXFP4 && kv_fmt != CSA2_KV_E4M3_16) return CSA2_ERR_UNSUPPORTED;
    if (Hm < 16 || Hm % 16) return Hm < 1 ? CSA2_ERR_INVALID_ARG : CSA2_ERR_UNSUPPORTED;
    if (K < 1 || K > kMaxK) return K < 1 ? CSA2_ERR_INVALID_ARG : CSA2_ERR_UNSUPPORTED;
    if (!(softmax_scale > 0.0f) || !std::isfinite(softmax_scale)) return CSA2_ERR_INVALID_ARG;
    if ((st = check_swa(batch, swa))) return st;
    if (ws && ((uintptr_t)ws & 255)) return CSA2_ERR_WORKSPACE;
    AttnLaunch a{batch, g, Hm, q_bf16, kv_fp4, kv_sc, idx, K, swa_rows, swa, softmax_scale, nullptr, lse, ws,
                 ws ? ws_bytes : 0, kv_fmt};
    a.rope_cs = rope_cs;
    a.out16 = out_bf16;
    hipError_t e = launch_sparse_attn(a, stream);
    return e == hipSuccess ? CSA2_OK : hip_fail(e);
}

CSA2_API csa2_status csa2_layer_chain(const csa2_batch* batch, const csa2_chain_params* p, int32_t n_layers,
                                      const csa2_layer* layers, const csa2_swa_layout* swa, int32_t* pool_blocks,
                                      int32_t* pool_pos, int32_t* pool_count, void* ws, size_t ws_bytes,
                                      hipStream_t stream) {
    Geometry g;
    csa2_status st = batch_geometry(batch, &g);
    if (st) return st;
    if (!p || !layers || n_layers < 1) return CSA2_ERR_INVALID_ARG;
    if (p->H != 32 && p->H != 64) return CSA2_ERR_UNSUPPORTED;
    if (p->Hm < 16 || p->Hm % 16) return CSA2_ERR_UNSUPPORTED;
    if (p->K < 1 || p->K > kMaxK) return p->K < 1 ? CSA2_ERR_INVALID_ARG : CSA2_ERR_UNSUPPORTED;
    if (p->block != 8) return CSA2_ERR_UNSUPPORTED;
    if (p->max_blocks < 1 || p->max_blocks > kMaxK) return CSA2_ERR_UNSUPPORTED;
    if (!(p->softmax_scale > 0.0f) || !std::isfinite(p->softmax_scale)) return CSA2_ERR_INVALID_ARG;
    if ((st = check_swa(batch, swa))) return st;
    // static checks of the schedule: every attending layer has main KV, every
    // REUSE layer has indices, at most one layer builds the pool
    bool have_kv = false, have_idx = false;
    bool src_mx = false;  // the latest Full layer's indexer K carries 32-channel scales
    int pool_layers = 0;
    for (int l = 0; l < n_layers; ++l) {
        const csa2_layer& L = layers[l];
        if (!L.q_main || !L.swa || !L.out) return CSA2_ERR_INVALID_ARG;
        switch (L.mode) {
            case CSA2_MODE_SWA_ONLY: break;
            case CSA2_MODE_FULL:
                if (!L.kv_fp4 || !L.kv_sc || !L.k_fp4 || !L.k_sc || !L.q_idx || !L.q_sc || !L.w) return CSA2_ERR_INVALID_ARG;
                if (L.q_fmt != CSA2_Q_FP4 && L.q_fmt != CSA2_Q_FP8 && L.q_fmt != CSA2_Q_MXFP4) return CSA2_ERR_INVALID_ARG;
                src_mx = L.q_fmt == CSA2_Q_MXFP4;
                if (L.kv_fmt != CSA2_KV_MXFP4 && L.kv_fmt != CSA2_KV_E4M3_16) return CSA2_ERR_UNSUPPORTED;
                have_kv = have_idx = true;
                if (L.flags & CSA2_LAYER_BUILD_POOL) ++pool_layers;
                break;
            case CSA2_MODE_REINDEX:
                if (!have_kv || !L.q_idx || !L.q_sc || !L.w) return CSA2_ERR_INVALID_ARG;
                if (L.q_fmt == CSA2_Q_FP8) return CSA2_ERR_UNSUPPORTED;  // pool scoring runs on FP4 queries
                if (L.q_fmt != CSA2_Q_FP4 && L.q_fmt != CSA2_Q_MXFP4) return CSA2_ERR_INVALID_ARG;
                if ((L.q_fmt == CSA2_Q_MXFP4) != src_mx) return CSA2_ERR_INVALID_ARG;  // the K's scale layout
                have_idx = true;
                break;
            case CSA2_MODE_REUSE:
                if (!have_idx) return CSA2_ERR_INVALID_ARG;
                break;
            default: return CSA2_ERR_INVALID_ARG;
        }
    }
    if (pool_layers > 1) return CSA2_ERR_INVALID_ARG;
    const ChainWs cw = chain_ws(g, p->K, p->block, p->max_blocks);
    if ((st = check_ws(ws, ws_bytes, cw.total))) return st;
    char* base = (char*)ws;
    float* scores = (float*)(base + cw.scores);
    float* pscores = (float*)(base + cw.pool_scores);
    char* pws = base + cw.pool_ws;
    int32_t* idx_cur = (int32_t*)(base + cw.idx_cur);
    int32_t* idx_empty = (int32_t*)(base + cw.idx_empty);
    uint32_t* tmax = (uint32_t*)(base + cw.tiles);
    uint32_t* tbound = (uint32_t*)(base + cw.tiles + al256((size_t)g.total_q * (size_t)cw.tstride * 4));
    char* po = base + cw.pool_out;
    int32_t* pb = pool_blocks ? pool_blocks : (int32_t*)po;
    po += al256((size_t)g.total_q * p->max_blocks * 4);
    int32_t* pp = pool_pos ? pool_pos : (int32_t*)po;
    po += al256((size_t)g.total_q * p->max_blocks * p->block * 4);
    int32_t* pc = pool_count ? pool_count : (int32_t*)po;
    const int64_t nb = (g.max_entries + p->block - 1) / p->block;
    const size_t bsc_bytes = al256((size_t)g.total_q * (size_t)(nb > 0 ? nb : 1) * 4);
    void* topk_ws = pws + bsc_bytes;
    const int pool_stride = p->max_blocks * p->block;

    hipError_t e;
    const int64_t nidx = (int64_t)g.total_q * p->K;
    bool any_swa_only = false;
    for (int l = 0; l < n_layers; ++l) any_swa_only |= layers[l].mode == CSA2_MODE_SWA_ONLY;
    if (any_swa_only) {  // the empty index list SWA-only layers attend with
        hipLaunchKernelGGL(k_fill_i32, dim3((unsigned)((nidx + 255) / 256 < 2048 ? (nidx + 255) / 256 : 2048)),
                           dim3(256), 0, stream, idx_empty, nidx, -1);
        if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e);
    }

    const csa2_layer* src = nullptr;  // latest Full layer (main KV + indexer K)
    bool pool_built = false;
    bool scan_timed = false;  // the caller's scan events go round the first Full layer's scan
    for (int l = 0; l < n_layers; ++l) {
        const csa2_layer& L = layers[l];
        const int32_t* use_idx = idx_cur;
        if (L.mode == CSA2_MODE_FULL || L.mode == CSA2_MODE_REINDEX) {
            const bool full = L.mode == CSA2_MODE_FULL;
            if (full) {
                src = &L;
                pool_built = false;
            }
            const bool on_pool = !full && pool_built;
            const bool build_pool = full && (L.flags & CSA2_LAYER_BUILD_POOL);
            if (full && local_scan_ok(g, L.q_fmt)) {
                // decode scan: per-chunk candidate lists and the rows' histograms
                // instead of score rows (plus the block maxima of the pool)
                const int ch = local_chunk(g);
                const int64_t mc = (g.max_entries + ch - 1) / ch;
                LocalOut lo{};
                lo.lists = (uint64_t*)scores;
                lo.counts = (uint32_t*)((char*)scores + al256(local_lists_bytes(g)));
                lo.bscores = build_pool ? (float*)pws : nullptr;
                lo.bstride = nb > 0 ? nb : 1;
                lo.max_chunks = (int)(mc > 0 ? mc : 1);
                lo.chunk = ch;
                lo.K = p->K;
                lo.block = p->block;
                // rows of few chunks: one kernel selects from the lists alone
                // (with the chunks' bounds); longer rows: the scan also fills
                // the rows' histograms, and the lists are filtered by many
                // workgroups first
                const bool fused_topk =
                    lo.max_chunks <= kListChunks && (int64_t)lo.max_chunks * lo.chunk <= kFusedTopkEntries;
                if (fused_topk) lo.lbins = (uint32_t*)((char*)lo.counts + al256(local_counts_bytes(g)));
                if (!fused_topk && (e = clear_topk_ws(topk_ws, g.total_q, true, stream)) != hipSuccess)
                    return hip_fail(e);
                ScoreLaunch sa{batch, g, p->H, L.q_fmt, (const uint8_t*)L.q_idx, L.q_sc, L.w, L.k_fp4, L.k_sc,
                               nullptr, 0, nullptr, 0, fused_topk ? nullptr : topk_ws_hist(topk_ws), &lo};
                if ((e = timed_scan(sa, p, &scan_timed, stream)) != hipSuccess) return hip_fail(e);
                if ((e = fused_topk ? launch_topk_fused(batch, g, lo, idx_cur, topk_ws, stream)
                                    : launch_topk_local(batch, g, lo, idx_cur, topk_ws, stream)) != hipSuccess)
                    return hip_fail(e);
                if (build_pool) {  // after the Top-K: the pool's selection reuses its workspace
                    PoolLaunch pa{};
                    pa.b = batch;
                    pa.g = g;
                    pa.block = p->block;
                    pa.max_blocks = p->max_blocks;
                    pa.blocks = pb;
                    pa.pool_pos = pp;
                    pa.pool_count = pc;
                    pa.bscores = (float*)pws;
                    pa.bstride = nb > 0 ? nb : 1;
                    pa.topk_ws = topk_ws;
                    pa.bscores_ready = true;
                    if ((e = launch_block_pool(pa, stream)) != hipSuccess) return hip_fail(e);
                    pool_built = true;
                }
            } else {
                // the score kernel builds the Top-K histogram when it can (FP4 queries,
                // at most 4 rows per sequence or a candidate list) and the rows are too
                // long for the one-workgroup selection; the Top-K pass then starts
                // from it.  A pool built from these scores needs its own pass.
                const int64_t slots = on_pool ? (int64_t)pool_stride : g.max_entries;
                const bool fused = L.q_fmt != CSA2_Q_FP8 && (on_pool || g.max_q_per_seq <= 4) && slots > kRowSelMax;
                if (fused && (e = clear_topk_ws(topk_ws, g.total_q, true, stream)) != hipSuccess) return hip_fail(e);
                ScoreLaunch sa{batch, g, p->H, L.q_fmt, (const uint8_t*)L.q_idx, L.q_sc, L.w, src->k_fp4, src->k_sc,
                               on_pool ? pp : nullptr, on_pool ? pool_stride : 0, on_pool ? pscores : scores,
                               on_pool ? (int64_t)pool_stride : (g.max_entries > 0 ? g.max_entries : 1),
                               fused ? topk_ws_hist(topk_ws) : nullptr};
                // a prefill scorer also records its tiles' maxima, which bound the
                // Top-K, and the block maxima a pool built here selects from
                const bool tiles = !on_pool && prefill_scorer(g, L.q_fmt);
                if (tiles) {
                    sa.tmax = tmax;
                    sa.tstride = cw.tstride;
                    if (build_pool && p->block == kPoolBlock && L.q_fmt != CSA2_Q_FP8) {
                        sa.bmax = (float*)pws;
                        sa.bstride = nb > 0 ? nb : 1;
                    }
                }
                if ((e = full ? timed_scan(sa, p, &scan_timed, stream) : launch_index_score(sa, stream)) != hipSuccess)
                    return hip_fail(e);
                TopkLaunch ta{};
                ta.b = batch;
                ta.g = g;
                ta.scores = on_pool ? pscores : scores;
                ta.stride = on_pool ? (int64_t)pool_stride : (g.max_entries > 0 ? g.max_entries : 1);
                ta.max_slots = on_pool ? pool_stride : g.max_entries;
                ta.cand = on_pool ? pp : nullptr;
                ta.cand_stride = on_pool ? pool_stride : 0;
                ta.cand_count = on_pool ? pc : nullptr;
                ta.block_mode = 0;
                ta.block = 1;
                ta.K = p->K;
                ta.idx = idx_cur;
                ta.ws = topk_ws;
                ta.hist = fused ? topk_ws_hist(topk_ws) : nullptr;
                if (tiles) {
                    ta.tmax = tmax;
                    ta.tstride = cw.tstride;
                    ta.tb = tbound;
                }
                if ((e = launch_topk(ta, stream)) != hipSuccess) return hip_fail(e);
                // the pool runs its own selection in the same workspace: after the Top-K
                if (build_pool) {
                    PoolLaunch pa{};
                    pa.b = batch;
                    pa.g = g;
                    pa.scores = scores;
                    pa.stride = g.max_entries > 0 ? g.max_entries : 1;
                    pa.block = p->block;
                    pa.max_blocks = p->max_blocks;
                    pa.blocks = pb;
                    pa.pool_pos = pp;
                    pa.pool_count = pc;
                    pa.bscores = (float*)pws;
                    pa.bstride = nb > 0 ? nb : 1;
                    pa.topk_ws = topk_ws;
                    pa.bscores_ready = sa.bmax != nullptr;  // the scorer wrote the block maxima
                    if ((e = launch_block_pool(pa, stream)) != hipSuccess) return hip_fail(e);
                    pool_built = true;
                }
            }
        } else if (L.mode == CSA2_MODE_SWA_ONLY) {
            use_idx = idx_empty;
        }
        const uint8_t* kv = src ? src->kv_fp4 : nullptr;
        const uint8_t* kvs = src ? src->kv_sc : nullptr;
        if (!kv) {  // SWA-only layers before any Full layer: no entry is read
            kv = (const uint8_t*)L.swa;
            kvs = (const uint8_t*)L.swa;
        }
        AttnLaunch aa{batch, g, p->Hm, L.q_main, kv, kvs, use_idx, p->K, L.swa, swa, p->softmax_scale, L.out, L.lse,
                      base + cw.attn, cw.attn_bytes, src ? src->kv_fmt : CSA2_KV_MXFP4};
        if ((e = launch_sparse_attn(aa, stream)) != hipSuccess) return hip_fail(e);
        if (L.idx_out) {
            if ((e = hipMemcpyAsync(L.idx_out, use_idx, (size_t)nidx * 4, hipMemcpyDeviceToDevice, stream)) != hipSuccess)
                return hip_fail(e);
        }
    }
    return CSA2_OK;
}

}  // extern "C"
