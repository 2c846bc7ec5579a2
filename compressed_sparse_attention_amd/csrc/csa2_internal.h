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
constexpr int kHistBins = 4096;        // top 12 value bits of a non-negative binary32 score (bits 30..19)
constexpr int kCandCap = 8192;         // per-row candidate capacity of the fast Top-K path
constexpr int kMaxK = 2048;

// Per-row state of the Top-K selection, in the workspace.
struct RowSel {
    uint32_t n;        // slots taking part
    uint32_t kk;       // min(K, n)
    uint32_t bin;      // threshold bin (candidates have bin >= this)
    uint32_t cnt;      // candidates collected (may exceed kCandCap -> fallback)
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
};
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
};
size_t topk_ws_bytes(int total_q);
// zero the histogram and row state of a Top-K workspace (done by launch_topk
// itself unless the caller filled the histogram beforehand)
hipError_t clear_topk_ws(void* ws, int total_q, bool hist_too, hipStream_t s);
uint32_t* topk_ws_hist(void* ws);
hipError_t launch_topk(const TopkLaunch& a, hipStream_t s);

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
    const uint16_t* swa;
    const csa2_swa_layout* sw;
    float scale;
    float* out;
    float* lse;
};
hipError_t launch_sparse_attn(const AttnLaunch& a, hipStream_t s);
hipError_t launch_gather_dequant(const csa2_batch* b, Geometry g, const uint8_t* kv, const uint8_t* kv_sc,
                                 const int32_t* idx, int K, uint16_t* out, hipStream_t s);

}  // namespace csa2
