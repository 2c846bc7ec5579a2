// Internal declarations of libcsa2 (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/csa2.h"

namespace csa2 {

// ---------------------------------------------------------------------------
// Vector types used as MFMA operands on gfx950.
// ---------------------------------------------------------------------------
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef short v4s __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kHistBins = 4096;        // bits 30..19 of a non-negative binary32 score; negatives in bin 0
constexpr int kCandCap = 8192;         // per-row candidate capacity of the fast Top-K path
constexpr int kMaxK = 2048;

// Per-row state of the Top-K selection, in the workspace.
struct RowSel {
    uint32_t n;        // slots taking part
    uint32_t kk;       // min(K, n)
    uint32_t bin;      // threshold bin (candidates have bin >= this)
    uint32_t cnt;      // candidates collected (may exceed kCandCap -> fallback)
    uint32_t above;    // keys in the bins above the threshold bin (all of them win)
    uint32_t lb;       // 1: `bin` is only a lower bound of the threshold bin (candidates hold every
                       //    key from it up; the selection starts from the top key bit)
    uint32_t pad[2];
};

struct Geometry {
    int n_seq, total_q, ratio;
    int64_t max_entries;  // max N_b
    int max_q_per_seq;    // max T_b
};

// Visible entries of a sequence with n entries for a query at token t.
__host__ __device__ inline int64_t visible_count(int64_t n, int64_t t, int m) {
    if (t < 0) return 0;
    int64_t v = (t + 1) / m;
    return v < n ? v : n;
}

// ---------------------------------------------------------------------------
// Selection order shared by the scan and the Top-K passes.  A score's bit
// pattern maps to an unsigned key that orders like the value for every
// binary32 but NaN (non-negative: set the sign bit; negative: invert all
// bits; -0 first becomes +0), so -inf < negatives < 0 < positives, and
//     key64 = (key << 32) | (0xFFFFFFFF - position)
// is unique per position and orders exactly like (score desc, position asc).
// The histograms have 4096 bins: a non-negative score's bits 30..19, with
// every negative score (and -inf) in bin 0.  Keys of a bin b >= 1 share their
// top 13 bits, b + 4096, so a selection inside such a bin starts at bit 51;
// bin 0 mixes signs, and a selection that starts there runs from the top bit.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t score_key(float s) {
    uint32_t u = __float_as_uint(s);
    u = u == 0x80000000u ? 0u : u;  // -0 equals +0: the same key, ties by position
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ uint32_t key_bin(uint32_t key) { return key >= 0x80000000u ? (key - 0x80000000u) >> 19 : 0u; }
__device__ __forceinline__ uint32_t key64_bin(uint64_t x) { return key_bin((uint32_t)(x >> 32)); }

// A workgroup barrier that orders LDS only: the fences cover the local address
// space, so the barrier waits for this wave's LDS operations but leaves its
// global loads in flight (a plain __syncthreads() waits for those as well,
// which defeats a prefetch issued ahead of it).  For kernels whose waves share
// data through LDS only.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ uint64_t composite(uint32_t key, uint32_t slot) {
    return ((uint64_t)key << 32) | (uint64_t)(0xFFFFFFFFu - slot);
}

// Inclusive scan of one value per thread over a 256-thread workgroup: a
// shuffle scan inside each wave, then the wave totals through LDS.  Every
// thread of the workgroup calls it.
__device__ inline uint32_t block_scan_256(uint32_t v, uint32_t* wtot) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t u = __shfl_up(v, off);
        if (lane >= off) v += u;
    }
    if (lane == 63) wtot[wave] = v;
    __syncthreads();
    for (int w2 = 0; w2 < wave; ++w2) v += wtot[w2];
    return v;
}

// Bin counts of a histogram in plain 32-bit words, or packed two 16-bit
// counts per word (bin 2i in the low half of word i).
struct PlainBins {
    const uint32_t* h;
    __device__ uint32_t operator()(int b) const { return h[b]; }
    // bins lo .. lo+15 (lo a multiple of 16) in four 16-byte loads
    __device__ void load16(int lo, uint32_t* c) const {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint4 v = *reinterpret_cast<const uint4*>(h + lo + 4 * i);
            c[4 * i] = v.x;
            c[4 * i + 1] = v.y;
            c[4 * i + 2] = v.z;
            c[4 * i + 3] = v.w;
        }
    }
};
struct PackedBins {
    const uint32_t* h;
    __device__ uint32_t operator()(int b) const { return (h[b >> 1] >> (16 * (b & 1))) & 0xFFFFu; }
    // bins lo .. lo+15 (lo a multiple of 16) in two 16-byte loads
    __device__ void load16(int lo, uint32_t* c) const {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint4 v = *reinterpret_cast<const uint4*>(h + (lo >> 1) + 4 * i);
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                c[8 * i + 2 * j] = w[j] & 0xFFFFu;
                c[8 * i + 2 * j + 1] = w[j] >> 16;
            }
        }
    }
};

// Block-wide (256 threads): the bin that holds the kk-th largest key; every
// thread returns it; kHistBins when kk == 0.  found[0..1] (LDS) end up holding
// the bin and the count of keys in the bins above it.  `found` and `wtot` are
// LDS scratch; a caller that calls it again must pass a barrier first.
template <class Bins>
__device__ inline uint32_t threshold_bin(Bins h, uint32_t kk, uint32_t* wtot, uint32_t* found) {
    const int t = threadIdx.x;
    // thread t owns bins [4096 - 16(t+1), 4096 - 16t), i.e. thread 0 the top bins
    const int hi = kHistBins - 16 * t;
    uint32_t up[16], c[16];  // up[i] = bin hi - 16 + i, c[i] = bin hi - 1 - i
    h.load16(hi - 16, up);
    uint32_t s = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        c[i] = up[15 - i];
        s += c[i];
    }
    if (t == 0) {
        found[0] = kk == 0 ? (uint32_t)kHistBins : 0u;
        found[1] = 0;
    }
    const uint32_t incl = block_scan_256(s, wtot);
    const uint32_t before = incl - s;
    if (kk > 0 && before < kk && kk <= incl) {
        uint32_t acc = before;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if (acc + c[i] >= kk) {
                found[0] = (uint32_t)(hi - 1 - i);
                found[1] = acc;
                break;
            }
            acc += c[i];
        }
    }
    __syncthreads();
    return found[0];
}

// The same search for two ranks k1 and k2 at once (k2 == 0: not searched):
// returns the bin of the k1-th largest key and leaves that of the k2-th in
// *bin2 (kHistBins when the rank is 0).  found[0..3] is LDS scratch.
template <class Bins>
__device__ inline uint32_t threshold_bin2(Bins h, uint32_t k1, uint32_t k2, uint32_t* wtot, uint32_t* found,
                                          uint32_t* bin2) {
    const int t = threadIdx.x;
    const int hi = kHistBins - 16 * t;
    uint32_t up[16], c[16];
    h.load16(hi - 16, up);
    uint32_t s = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        c[i] = up[15 - i];
        s += c[i];
    }
    if (t == 0) {
        found[0] = k1 == 0 ? (uint32_t)kHistBins : 0u;
        found[2] = k2 == 0 ? (uint32_t)kHistBins : 0u;
    }
    const uint32_t incl = block_scan_256(s, wtot);
    const uint32_t before = incl - s;
    const uint32_t ks[2] = {k1, k2};
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const uint32_t kk = ks[r];
        if (kk > 0 && before < kk && kk <= incl) {
            uint32_t acc = before;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                if (acc + c[i] >= kk) {
                    found[2 * r] = (uint32_t)(hi - 1 - i);
                    break;
                }
                acc += c[i];
            }
        }
    }
    __syncthreads();
    *bin2 = found[2];
    return found[0];
}

// binary32 -> bf16 to nearest even.  Finite values and infinities: adding
// 0x7FFF plus the kept part's lowest bit carries exactly when the dropped 16
// bits exceed half a unit, or equal it with an odd kept part; a carry out of
// the largest finite value gives infinity.  A NaN stays a NaN: its sign and
// leading payload bits are kept and the quiet bit is set (the addition alone
// could carry a NaN into an infinity or the other sign).
__host__ __device__ inline uint32_t bf16_rne(float f) {
    uint32_t u;
    __builtin_memcpy(&u, &f, 4);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x0040u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}


// ---------------------------------------------------------------------------
// Per-chunk candidate lists written by the decode scan in place of the full
// score rows.  A chunk is a run of positions one scan workgroup covers.  For
// each (row, chunk) the scan keeps every visible position whose bin is at or
// above the bin of the chunk's min(K, visible)-th largest score; the row's
// Top-K lies in the union of its chunks' lists, because a position ranked
// among the row's first K is ranked among its chunk's first K.  Lists hold
// key64 values in position order.
// ---------------------------------------------------------------------------
struct LocalOut {
    uint64_t* lists;     // [total_q][max_chunks][chunk]
    uint32_t* counts;    // [total_q][max_chunks]; written for chunks that hold positions
    float* bscores;      // nullable: block maxima [total_q][bstride] for the block pool
    uint32_t* lbins;     // nullable: [total_q][max_chunks], for each chunk whose positions are all
                         // visible, the bin of its ceil(K / such chunks)-th largest score
    int64_t bstride;
    int max_chunks;
    int chunk;
    int K;
    int block;
};

// positions per decode-scan workgroup: 4 waves x 16 tiles of 64, halved for
// the 4-row scan when it keeps its rows' scores on chip (LDS budget)
constexpr int decode_chunk(int tq, bool local) { return (local && tq > 1) ? 2048 : 4096; }
// the scan writes local lists for FP4 queries and at most 4 rows per sequence
inline bool local_scan_ok(const Geometry& g, int q_fmt) { return q_fmt != CSA2_Q_FP8 && g.max_q_per_seq <= 4; }
inline int local_chunk(const Geometry& g) { return decode_chunk(g.max_q_per_seq <= 1 ? 1 : 4, true); }
inline size_t local_lists_bytes(const Geometry& g) {
    const int ch = local_chunk(g);
    const int64_t mc = (g.max_entries + ch - 1) / ch;
    return (size_t)g.total_q * (size_t)(mc > 0 ? mc : 1) * ch * 8;
}
inline size_t local_counts_bytes(const Geometry& g) {
    const int ch = local_chunk(g);
    const int64_t mc = (g.max_entries + ch - 1) / ch;
    return (size_t)g.total_q * (size_t)(mc > 0 ? mc : 1) * 4;
}

// ---------------------------------------------------------------------------
// Kernel launchers (defined in the .hip files).  All return hipError_t of
// the launch; shapes were validated by the caller.
// ---------------------------------------------------------------------------
struct ScoreLaunch {
    const csa2_batch* b;
    Geometry g;
    int H, q_fmt;
    const uint8_t* q;
    const uint8_t* q_sc;
    const float* w;
    const uint8_t* k;
    const uint8_t* k_sc;
    const int32_t* cand;
    int cand_stride;
    float* scores;
    int64_t stride;
    uint32_t* hist;             // nullable: [total_q][kHistBins], zeroed by the caller
    const LocalOut* local;      // nullable: decode scan writes per-chunk candidate lists, not scores
    hipEvent_t ev_begin = nullptr, ev_end = nullptr;  // optional: stamped by the score kernel's dispatch
    // nullable, prefill scorers only (prefill_scorer): the key (score_key) of
    // the largest score of each row's kTile-slot tile, [total_q][tstride],
    // written for the tiles that hold a slot the row sees
    uint32_t* tmax = nullptr;
    int64_t tstride = 0;
    // nullable, the FP4 prefill scorer only (E4M3 queries: an error): the
    // largest score of each kPoolBlock-slot block of a row, [total_q][bstride]
    // (what k_block_max computes), written for the blocks that hold a slot
    // the row sees
    float* bmax = nullptr;
    int64_t bstride = 0;
};
// slots per block of the block pool the prefill scorers' maxima serve
constexpr int kPoolBlock = 8;
// slots per tile of the prefill scorers' tile maxima
constexpr int kTile = 64;
// score rows come from a prefill scorer (many query rows, or E4M3 queries)
// rather than from the decode scan
inline bool prefill_scorer(const Geometry& g, int q_fmt) { return q_fmt == CSA2_Q_FP8 || g.max_q_per_seq > 4; }
hipError_t launch_index_score(const ScoreLaunch& a, hipStream_t s);

struct TopkLaunch {
    const csa2_batch* b;
    Geometry g;
    const float* scores;
    int64_t stride;
    int64_t max_slots;          // upper bound of slots per row
    const int32_t* cand;        // NULL: slot = position
    int cand_stride;
    const int32_t* cand_count;  // with cand
    int block_mode;             // 1: slots are blocks of `block` positions over vis (n = ceil(vis/block))
    int block;
    int K;
    int32_t* idx;               // [total_q][K]
    void* ws;
    const uint32_t* hist;       // nullable: histogram of the scores made with them (skips the histogram pass)
    // nullable: the scores' tile maxima (ScoreLaunch::tmax) and room for one
    // bound per row: rows of at least K tiles are then bounded by their K-th
    // largest tile maximum and only the tiles that reach it are read
    const uint32_t* tmax = nullptr;
    int64_t tstride = 0;
    uint32_t* tb = nullptr;
};
// Rows of at most kRowSelMax slots are selected by one workgroup each, from
// their scores alone (a histogram made with the scores is not used)
constexpr int kRowSelMax = 16384;
size_t topk_ws_bytes(int total_q);
// zero the histogram and row state of a Top-K workspace (done by launch_topk
// itself unless the caller filled the histogram beforehand)
hipError_t clear_topk_ws(void* ws, int total_q, bool hist_too, hipStream_t s);
uint32_t* topk_ws_hist(void* ws);
hipError_t launch_topk(const TopkLaunch& a, hipStream_t s);
// Top-K from a scan's per-chunk lists and its histogram (in the workspace,
// cleared before the scan together with the row state)
hipError_t launch_topk_local(const csa2_batch* b, const Geometry& g, const LocalOut& lo, int32_t* idx, void* ws,
                             hipStream_t s);

// The Top-K from a scan's per-chunk lists and the chunks' bounds, without a
// histogram from the scan: many workgroups keep the list entries at or above
// the row's bound (in ws, a Top-K workspace), then one workgroup per row
// selects among them (or, when they do not fit, from the lists).  Correct for
// any list length up to kListChunks chunks per row; chosen for rows of at
// most kFusedTopkEntries entries (max_chunks * chunk), while longer rows take
// the scan's histogram (launch_topk_local).
constexpr int kListChunks = 1024;
constexpr int64_t kFusedTopkEntries = 262144;
hipError_t launch_topk_fused(const csa2_batch* b, const Geometry& g, const LocalOut& lo, int32_t* idx, void* ws,
                             hipStream_t s);

struct PoolLaunch {
    const csa2_batch* b;
    Geometry g;
    const float* scores;
    int64_t stride;
    int block, max_blocks;
    int32_t* blocks;
    int32_t* pool_pos;
    int32_t* pool_count;
    float* bscores;             // workspace [total_q][bstride]
    int64_t bstride;
    void* topk_ws;
    bool bscores_ready;         // the scan already wrote the block maxima
};
hipError_t launch_block_pool(const PoolLaunch& a, hipStream_t s);

struct AttnLaunch {
    const csa2_batch* b;
    Geometry g;
    int Hm;
    const uint16_t* q;
    const uint8_t* kv;
    const uint8_t* kv_sc;
    const int32_t* idx;
    int K;
    const void* swa;            // SWA rows in the layout's format (bf16 or MXFP8)
    const csa2_swa_layout* sw;
    float scale;
    float* out;
    float* lse;
    void* ws;                   // partial results when the key blocks are split (may be NULL)
    size_t ws_bytes;
    int kv_fmt;                 // CSA2_KV_* of kv_sc
    // fused RoPE and casts (csa2_sparse_attn_rope): q holds the query before
    // RoPE, rotated and cast on load; the output's rotated channels are turned
    // back and every channel cast to bf16 on store (out16)
    const float* rope_cs = nullptr;  // [total_q][32][2] cos, sin per pair
    uint16_t* out16 = nullptr;       // [total_q][Hm][512]
};

// RoPE pairs (448 + 2p, 449 + 2p), p < 32, of a head row (the append's and
// csa2_rope_cast's): (a, b) -> (a cos - b sin, a sin + b cos), each product
// and the sum or difference rounded to fp32; `sg` = -1 negates the angle.
__device__ __forceinline__ void rope_pair(float& a, float& b, float co, float si, float sg) {
#pragma clang fp contract(off)
    const float s = sg * si;  // exact negation
    const float x = a, y = b;
    a = x * co - y * s;
    b = x * s + y * co;
}
// key-block splits the attention would use, and the workspace they need
int attn_splits(const Geometry& g, int Hm, int K, int W);
size_t attn_ws_bytes(const Geometry& g, int Hm, int S);
hipError_t launch_sparse_attn(const AttnLaunch& a, hipStream_t s);
// Many rows: one workgroup per (row, 64 heads) when the grid has at least
// kAttnRowsMinWgs of them, two per CU (launch_sparse_attn dispatches to it)
constexpr int kAttnRowsMinWgs = 512;
inline bool attn_rows_ok(const Geometry& g, int Hm) {
    return Hm % 64 == 0 && (int64_t)g.total_q * (Hm / 64) >= kAttnRowsMinWgs;
}
hipError_t launch_sparse_attn_rows(const AttnLaunch& a, hipStream_t s);
hipError_t launch_rope_cast(int64_t n_rows, int heads, const float* in, const float* cs, int inverse, uint16_t* out,
                            hipStream_t s);
hipError_t launch_index_k_project(int64_t n, const float* x, const float* cs, const float* W, const int64_t* dst,
                                  int64_t rows, int mx, uint8_t* k_fp4, uint8_t* k_sc, hipStream_t s);
hipError_t launch_compress(int64_t n, int m, const float* c_tok, const float* z_tok, float* out, hipStream_t s);
hipError_t launch_kv_append(int64_t n, const float* x, const float* cs, const int64_t* dst, int64_t rows, int kv_fmt,
                            uint8_t* kv, uint8_t* kv_sc, hipStream_t s);
hipError_t launch_gather_dequant(const csa2_batch* b, Geometry g, int kv_fmt, const uint8_t* kv, const uint8_t* kv_sc,
                                 const int32_t* idx, int K, uint16_t* out, hipStream_t s);

}  // namespace csa2
