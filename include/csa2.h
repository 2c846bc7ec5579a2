/*
 * csa2.h -- C ABI of libcsa2.so: CSA2 sparse attention over a compressed global
 * KV cache, written for AMD Instinct MI355X (gfx950).
 *
 * The method is that of the report "DeepSeek-V4.1-Flash: Pushing the Limits of
 * KV Cache Compression": a lightweight indexer scores the cached main-KV
 * entries with indexer Q and indexer K and keeps the Top-K entries per query;
 * each query then attends to the selected entries together with the layer's
 * sliding-window KV (section 2.3).  Layers run in one of three modes -- Full,
 * Reindex, Reuse -- that share main KV, indexer K and Top-K indices across
 * layers (section 2.3.1); in the decoder the first Full layer also builds a
 * block pool that bounds where later Reindex layers search (section 2.3.2).
 *
 * Conventions for every call
 *   - Tensor pointers marked (device) are device memory owned by the caller.
 *     The library never allocates or frees device memory.  Scratch memory is a
 *     caller workspace of at least csa2_workspace_size() bytes, 256-byte aligned
 *     (csa2_topk_noalloc alone uses a static array in the library instead).
 *   - Pointers marked (host) are read on the host during the call only.
 *   - Calls are asynchronous on `stream`: they enqueue kernels and return.  The
 *     library never synchronises the host with the device.
 *   - Arguments are validated on the host first; a call that returns an error
 *     has enqueued nothing (CSA2_ERR_HIP excepted: a launch failed part-way).
 *   - No global mutable state other than csa2_topk_noalloc's scratch; calls
 *     are thread-safe.  Calls that share a workspace (or that scratch) must
 *     be ordered on one stream.
 *
 * Data formats (OCP Microscaling Formats v1.0, which the report names as
 * "OCP-standard MXFP4", section 2.4.4):
 *   E2M1  4-bit float, values +-{0, .5, 1, 1.5, 2, 3, 4, 6}; two per byte,
 *         element 2i in the low nibble of byte i.
 *   E8M0  8-bit power-of-two scale 2^(e-127); 255 (NaN) is not allowed.
 *   E4M3  OCP 8-bit float (bias 7, max 448, no infinities).
 *   bf16  the upper 16 bits of an IEEE binary32.
 * Layouts (entries of all sequences packed back to back; entry_off gives the
 * first entry of each sequence):
 *   main KV     kv_fp4 [total_entries][256] u8 (512 E2M1 latent channels)
 *               kv_sc  CSA2_KV_MXFP4:    [total_entries][16] u8 (one E8M0 per 32 channels)
 *                      CSA2_KV_E4M3_16:  [total_entries][32] u8 (one E4M3 per 16 channels: the
 *                      report's main-KV format, section 2.4.4, NVFP4's layout without its
 *                      second-level global scale)
 *   indexer K   k_fp4  [total_entries][64]  u8 (128 E2M1 channels)
 *               k_sc   [total_entries]      u8 (one E8M0 per row), or with CSA2_Q_MXFP4
 *                      [total_entries][4] u8 (one E8M0 per 32 channels)
 *   indexer q   CSA2_Q_FP4, CSA2_Q_MXFP4: [total_q][H][64] u8, CSA2_Q_FP8: [total_q][H][128] u8
 *               q_sc   [total_q][H] u8 (one E8M0 per head row), or with CSA2_Q_MXFP4
 *                      [total_q][H][4] u8 (one E8M0 per 32 channels)
 *               w      [total_q][H] f32 head weights
 *   main q      [total_q][Hm][512] bf16
 *   SWA KV      per layer, rows of sequence b at row_off[b], holding token
 *               positions pos0[b] .. pos0[b]+len[b]-1; by the layout's fmt:
 *               CSA2_SWA_BF16  [rows][512] bf16
 *               CSA2_SWA_MXFP8 [rows][528] u8: 512 E4M3 codes, then 16 E8M0
 *                              scales (one per 32 channels; OCP MXFP8, the
 *                              FP8 SWA cache of the report's section 2.4.4)
 *   indices     [total_q][K] i32 local entry positions, ascending, -1 padded
 */
#ifndef CSA2_H
#define CSA2_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(CSA2_BUILDING_LIBRARY)
#define CSA2_API __attribute__((visibility("default")))
#else
#define CSA2_API
#endif

typedef int32_t csa2_status;
#define CSA2_OK 0
#define CSA2_ERR_INVALID_ARG 1   /* null pointer, bad size, stride too small, inconsistent batch */
#define CSA2_ERR_UNSUPPORTED 2   /* a size this build does not implement (see each call) */
#define CSA2_ERR_WORKSPACE 3     /* workspace missing, misaligned or too small */
#define CSA2_ERR_HIP 4           /* a HIP launch failed; csa2_last_hip_error() has the code */
#define CSA2_ERR_SCRATCH 5       /* larger than the static scratch of an allocation-free call */

#define CSA2_Q_FP4 0
#define CSA2_Q_FP8 1
/* The report's indexer format (section 2.4.4: quantisation-aware FP4 indexer
 * queries and keys in OCP MXFP4): E2M1 queries and indexer K, both with one
 * E8M0 per 32 channels.  It sets the layout of q_sc and of the indexer K's
 * k_sc together. */
#define CSA2_Q_MXFP4 2

#define CSA2_KV_MXFP4 0    /* main-KV scales: E8M0 per 32 channels */
#define CSA2_KV_E4M3_16 1  /* main-KV scales: E4M3 per 16 channels */

#define CSA2_SWA_BF16 0
#define CSA2_SWA_MXFP8 1

#define CSA2_MODE_SWA_ONLY 0
#define CSA2_MODE_FULL 1
#define CSA2_MODE_REINDEX 2
#define CSA2_MODE_REUSE 3

#define CSA2_LAYER_BUILD_POOL 1  /* this Full layer builds the block pool (first decoder Full layer) */

/* Ragged batch.  Sequence b owns entries entry_off[b] .. entry_off[b+1]-1 of the
 * packed caches and query rows q_off[b] .. q_off[b+1]-1; query row r sits at
 * token position q_pos[r].  With compression ratio m (report 2.3: entry j is
 * built from tokens jm .. jm+m-1, no overlap) entry j is visible to a query at
 * token t iff (j+1)*m - 1 <= t; the visible entries are 0 .. vis-1 with
 * vis = min(N_b, floor((t+1)/m)).  The host arrays and the device arrays hold
 * the same values: the host copies size the launches, the kernels read the
 * device copies. */
typedef struct csa2_batch {
    int32_t n_seq;               /* >= 1 */
    int32_t total_q;             /* >= 1 */
    int32_t ratio;               /* compression ratio m >= 1 (1 decoder, 2 encoder) */
    int32_t reserved;
    const int64_t* h_entry_off;  /* (host)   [n_seq+1], non-decreasing, h_entry_off[0] = 0 */
    const int32_t* h_q_off;      /* (host)   [n_seq+1], non-decreasing, h_q_off[n_seq] = total_q */
    const int32_t* h_q_pos;      /* (host)   [total_q], >= 0 */
    const int64_t* d_entry_off;  /* (device) [n_seq+1] */
    const int32_t* d_q_off;      /* (device) [n_seq+1] */
    const int32_t* d_q_pos;      /* (device) [total_q] */
    const int32_t* d_row_seq;    /* (device) [total_q] sequence of each query row */
} csa2_batch;

/* Sliding-window KV layout, shared by every layer of a call (the rows
 * themselves are per layer).  Query row r of sequence b at token t attends to
 * SWA rows for tokens u in [max(s_b, t-W+1), t] (course notes "3. 通用基础设施"
 * section 3.2.2), s_b = replay start (0 when d_replay_s is NULL).  Every such
 * token must lie in [pos0[b], pos0[b]+len[b]); the host checks this. */
typedef struct csa2_swa_layout {
    int32_t window;              /* W >= 1 (128 in the report, section 4.2.1) */
    int32_t fmt;                 /* CSA2_SWA_BF16 or CSA2_SWA_MXFP8: the rows' format */
    const int64_t* h_row_off;    /* (host)   [n_seq] first row of sequence b */
    const int32_t* h_pos0;       /* (host)   [n_seq] token position of that row */
    const int32_t* h_len;        /* (host)   [n_seq] rows present */
    const int32_t* h_replay_s;   /* (host)   [n_seq] or NULL */
    const int64_t* d_row_off;    /* (device) [n_seq] */
    const int32_t* d_pos0;       /* (device) [n_seq] */
    const int32_t* d_replay_s;   /* (device) [n_seq] or NULL */
} csa2_swa_layout;

/* ---- index score ---------------------------------------------------------
 * Lightning-indexer scores (report 2.3; Full mode 2.3.1 scores every visible
 * entry, Reindex mode rescores the shared indexer K with its own q):
 *   score(r, j) = 2^(k_sc[j]-127) * sum_{h=0..H-1} w[r,h] * ReLU(d_h * 2^(q_sc[r,h]-127))
 *   d_h = sum_c q[r,h,c] * k[j,c]   (exact: FP4 x FP4, and FP8 x FP4 for |q| <= 16)
 * With CSA2_Q_MXFP4 the scales sit inside the dot product and no per-entry
 * factor follows:
 *   score(r, j) = sum_h w[r,h] * ReLU(d_h),
 *   d_h = sum_b 2^(q_sc[r,h,b] + k_sc[j,b] - 254) * sum_{c in block b} q[r,h,c] * k[j,c]
 * which is exact while the four block exponents of a (head row, entry) pair
 * span few enough powers of two for d_h to fit binary32 (MX-quantised rows
 * span a few; rows far outside that may differ from the exact value in the
 * last bits).
 * The head sum is the binary32 chain acc = +0; acc = fmaf(w[r,h], ReLU(..), acc)
 * for h ascending, so scores are bit-reproducible.
 * cand == NULL: slot s of row r is entry s of its sequence; slots 0 .. N_b-1
 *   are written, -inf where the entry is not visible.
 * cand != NULL: slot s of row r is entry cand[r*cand_stride + s] (-1 = empty);
 *   slots 0 .. cand_stride-1 are written, -inf for empty or invisible slots.
 * q: [total_q][H][64] (CSA2_Q_FP4, CSA2_Q_MXFP4) or [total_q][H][128] (CSA2_Q_FP8)
 *   (device); q_sc and k_sc as the format sets them (layout table above).
 * scores: [total_q][score_stride] f32 (device); score_stride >= max N_b
 *   (cand == NULL) or >= cand_stride.
 * hist: NULL, or [total_q][4096] u32 (device, zeroed by the caller) that
 *   receives, per row, the count of written finite scores in each bin of bits
 *   30..19 (visible slots; with cand, the non-empty visible slots).  Passing it
 *   on to csa2_topk saves the Top-K pass its own histogram pass.  Not
 *   produced for CSA2_Q_FP8 queries in this build (the call then returns
 *   CSA2_ERR_UNSUPPORTED).
 * Supported: H in {32, 64}.  CSA2_Q_FP8 requires cand == NULL.  An unknown
 * q_fmt is CSA2_ERR_INVALID_ARG. */
CSA2_API csa2_status csa2_index_score(const csa2_batch* batch, int32_t H, int32_t q_fmt, const void* q,
                                      const uint8_t* q_sc, const float* w, const uint8_t* k_fp4,
                                      const uint8_t* k_sc, const int32_t* cand, int32_t cand_stride,
                                      float* scores, int64_t score_stride, uint32_t* hist, hipStream_t stream);

/* ---- RoPE and cast around attention ---------------------------------------
 * The report's kernel flow fuses RoPE, attention, RoPE and a cast: the query
 * is rotated before attention and the output's rotated part is turned back
 * after it.  For every head row of in [n_rows][heads][512] f32: channels
 * 448..511 in pairs (448 + 2p, 449 + 2p) rotated by the row's angle p
 * (rope_cs [n_rows][32][2] = cos, sin; inverse != 0 negates the angle), each
 * product and the sum or difference rounded to fp32, then every channel cast
 * to bf16 to nearest even into out_bf16 [n_rows][heads][512].
 * All pointers device, 16-byte aligned.  Errors: n_rows < 0, heads < 1, a
 * NULL or misaligned pointer with n_rows > 0: CSA2_ERR_INVALID_ARG. */
CSA2_API csa2_status csa2_rope_cast(int64_t n_rows, int32_t heads, const float* in, const float* rope_cs,
                                    int32_t inverse, uint16_t* out_bf16, hipStream_t stream);

/* ---- indexer-K projection --------------------------------------------------
 * Indexer K of new entries, projected from their main KV (reading note
 * "DeepSeek V4.1 Flash: Pushing the Limits of KV Cache Compression",
 * configuration section: indexer K comes directly from the main KV by a
 * projection; the report, section 2.4.4: FP4 indexer keys in OCP MXFP4):
 *   y[o] = sum_k x[i][k] W[k][o], o < 128, evaluated as the fp32 chain
 *          acc = +0; acc = fmaf(x[i][k], W[k][o], acc) for k = 0..511;
 *   row dst_row[i] of k_fp4 = E2M1(y / X) to nearest even, saturating at 6,
 *   X = 2^(floor(log2 amax) - 2) (at least 2^-127; 1 when amax = 0) over the
 *   row (q_fmt CSA2_Q_FP4 or CSA2_Q_FP8: k_sc [rows] u8) or over each 32
 *   channels (CSA2_Q_MXFP4: k_sc [rows][4] u8).
 * x: [n][512] f32 (device, 16-byte aligned), the entries' main KV before
 *   quantisation: after RoPE when rope_cs is NULL; before RoPE (the rows
 *   csa2_compress writes and csa2_kv_append takes) when rope_cs is given.
 * rope_cs: NULL, or [n][32][2] f32 (device, 16-byte aligned), the angles
 *   csa2_kv_append takes for the same entries; channels 448..511 of x are
 *   then turned first exactly as csa2_kv_append turns them (pair p =
 *   (448 + 2p, 449 + 2p), rounded products, no fused multiply-add).
 * W: [512][128] f32 (device, 16-byte aligned).
 * dst_row: [n] i64 (device); rows outside [0, n_rows) are skipped.
 * k_fp4: [n_rows][64] u8 (device, 16-byte aligned).
 * Errors: n < 0, an unknown q_fmt, a NULL pointer (rope_cs aside), a
 * misaligned pointer or n_rows < 1 with n > 0: CSA2_ERR_INVALID_ARG.  n == 0
 * does nothing. */
CSA2_API csa2_status csa2_index_k_project(int64_t n, const float* x, const float* rope_cs, const float* W,
                                          const int64_t* dst_row, int64_t n_rows, int32_t q_fmt, uint8_t* k_fp4,
                                          uint8_t* k_sc, hipStream_t stream);

/* ---- compressor -----------------------------------------------------------
 * The CSA2 compressor: m consecutive tokens become one global entry.  The
 * reading note "DeepSeek V4.1 Flash: Pushing the Limits of KV Cache
 * Compression" gives the KV rows C = H W^KV and their compression weights
 * Z = H W^Z; CSA2 drops V4's overlapping windows and absolute position
 * embedding, so entry j takes tokens jm .. jm + m - 1.  Reading: per channel,
 *   out[j][c] = sum_i exp(Z[jm+i][c]) C[jm+i][c] / sum_i exp(Z[jm+i][c])
 * (the softmax over the entry's tokens), in fp32 with the largest Z of the
 * channel subtracted first.
 * c_tok, z_tok: [n_entries * m][512] f32 (device, 16-byte aligned).
 * out: [n_entries][512] f32 (device, 16-byte aligned): the entries before
 *   RoPE, as csa2_kv_append takes them.
 * Errors: n_entries < 0, a NULL or misaligned pointer with n_entries > 0:
 * CSA2_ERR_INVALID_ARG; m outside 1..16: CSA2_ERR_UNSUPPORTED. */
CSA2_API csa2_status csa2_compress(int64_t n_entries, int32_t m, const float* c_tok, const float* z_tok, float* out,
                                   hipStream_t stream);

/* ---- cache append ---------------------------------------------------------
 * Writes new main-KV entries into their cache rows the way the report stores
 * them (section 2.4.4: the cache is quantised after RoPE, all 512 channels
 * including the rotated part; section 4.2.1: the RoPE part is 64 dimensions).
 * Entry i (i < n):
 *   1. rotation of channels 448..511: pair p = (448 + 2p, 449 + 2p), p < 32,
 *      (a, b) -> (a cos - b sin, a sin + b cos) with (cos, sin) =
 *      rope_cs[i][p][0..1], each product and the sum or difference rounded
 *      to fp32 (no fused multiply-add);
 *   2. quantisation into row dst_row[i] of kv_fp4 / kv_sc, by kv_fmt:
 *      CSA2_KV_E4M3_16: per 16 channels X = E4M3(fl32(amax / 6)) to nearest
 *        even (2^-9 where that is 0), kv_sc [rows][32];
 *      CSA2_KV_MXFP4: per 32 channels X = 2^(floor(log2 amax) - 2), at least
 *        2^-127 (1 for an all-zero block), kv_sc [rows][16] E8M0;
 *      codes E2M1(fl32(x / X)) to nearest even, saturating at 6, element 2c in
 *      the low nibble of byte c of the 256-byte row.
 * x: [n][512] f32 (device, 16-byte aligned), the entries' latents before RoPE.
 * rope_cs: [n][32][2] f32 (device, 16-byte aligned).
 * dst_row: [n] i64 (device); a row outside [0, n_rows) is skipped (the host
 *   cannot read it to check).  Two entries with one row race.
 * kv_fp4: [n_rows][256] u8 (device, 16-byte aligned); kv_sc as above.
 * Errors: n < 0, a NULL pointer or n_rows < 1 with n > 0, misaligned x,
 * rope_cs or kv_fp4: CSA2_ERR_INVALID_ARG; an unknown kv_fmt:
 * CSA2_ERR_UNSUPPORTED.  n == 0 does nothing. */
CSA2_API csa2_status csa2_kv_append(int64_t n, const float* x, const float* rope_cs, const int64_t* dst_row,
                                    int64_t n_rows, int32_t kv_fmt, uint8_t* kv_fp4, uint8_t* kv_sc,
                                    hipStream_t stream);

/* ---- Top-K ---------------------------------------------------------------
 * Per query row, the first min(K, n) slots under (score descending, entry
 * position ascending), written as entry positions in ascending order and -1
 * padded (report 2.3, "selects the Top-K entries for each query"; K = 512 in
 * section 4.2.1).  n = vis(row) when cand == NULL (slots are positions), else
 * n = cand_count[row] and slot s maps to position cand[row*cand_stride + s];
 * the first n candidate positions must be ascending.  Scores of the n slots
 * are ordered by value, negative ones and -inf included (-inf last); they
 * must not be NaN.
 * hist: NULL, or the histogram csa2_index_score wrote for exactly these scores
 *   (with cand, valid when the first cand_count slots are all non-empty and
 *   visible, as in a block pool).
 * idx: [total_q][K] i32 (device).  Supported: 1 <= K <= 2048.
 * Workspace: csa2_workspace_size(CSA2_WS_TOPK, ...). */
CSA2_API csa2_status csa2_topk(const csa2_batch* batch, const float* scores, int64_t score_stride,
                               const int32_t* cand, int32_t cand_stride, const int32_t* cand_count, int32_t K,
                               const uint32_t* hist, int32_t* idx, void* ws, size_t ws_bytes, hipStream_t stream);

/* ---- Top-K without allocation ----------------------------------------------
 * For callers that cannot allocate device memory or pass a workspace (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): csa2_topk with the same arguments and results, its workspace
 * taken from a static scratch array in the library's device code instead of
 * `ws`.  The array holds the workspace of at most 256 query rows (about
 * 20 MiB, held on every GPU the library runs on until the process ends);
 * a batch with more rows returns CSA2_ERR_SCRATCH and enqueues nothing.
 * The call allocates nothing; its first call on a device looks up the
 * array's device address (hipGetSymbolAddress) on the stream's device.
 * Every call on one GPU shares that GPU's array: calls that may overlap on
 * one GPU (different streams, or different host threads) race and must be
 * ordered by the caller.  The array keeps the last call's contents; the call
 * clears what must start at zero itself. */
CSA2_API csa2_status csa2_topk_noalloc(const csa2_batch* batch, const float* scores, int64_t score_stride,
                                       const int32_t* cand, int32_t cand_stride, const int32_t* cand_count, int32_t K,
                                       const uint32_t* hist, int32_t* idx, hipStream_t stream);

/* ---- block pool ----------------------------------------------------------
 * Hierarchical Sparse Indexer candidate pool (report 2.3.2; the reading note
 * "DeepSeek V4.1 Flash: Pushing the Limits of KV Cache Compression" states that
 * the pool and the Top-K are two independent selections from the same
 * position scores).  Blocks b cover positions [b*block, (b+1)*block), aligned
 * at 0; a block exists when it holds a visible position and its score is the
 * maximum score over its visible positions.  The first min(max_blocks, #blocks)
 * blocks under (block score descending, block ascending) are kept.
 * scores: Full-mode scores as csa2_index_score writes them (cand == NULL).
 * blocks:     [total_q][max_blocks] i32 ascending, -1 padded (device)
 * pool_pos:   [total_q][max_blocks*block] i32 visible positions of the kept
 *             blocks, ascending, -1 padded (device)
 * pool_count: [total_q] i32 (device)
 * Supported: block == 8, 1 <= max_blocks <= 2048.
 * Workspace: csa2_workspace_size(CSA2_WS_BLOCK_POOL, ...). */
CSA2_API csa2_status csa2_block_pool(const csa2_batch* batch, const float* scores, int64_t score_stride,
                                     int32_t block, int32_t max_blocks, int32_t* blocks, int32_t* pool_pos,
                                     int32_t* pool_count, void* ws, size_t ws_bytes, hipStream_t stream);

/* ---- gather + dequantise --------------------------------------------------
 * out[r][s][c] = E2M1(kv_fp4[e][c]) * scale(e, c) as bf16 (exact: at most six
 * significant bits), e = entry_off[seq(r)] + idx[r][s]; rows for idx == -1
 * are zero.  scale(e, c) = 2^(kv_sc[e][c/32]-127) for CSA2_KV_MXFP4 and
 * E4M3(kv_sc[e][c/16]) for CSA2_KV_E4M3_16.  Main KV is dequantised before
 * attention (report 2.4.4).
 * out_bf16: [total_q][K][512] (device).  Supported: 1 <= K <= 4096. */
CSA2_API csa2_status csa2_gather_dequant(const csa2_batch* batch, int32_t kv_fmt, const uint8_t* kv_fp4,
                                         const uint8_t* kv_sc, const int32_t* idx, int32_t K, uint16_t* out_bf16,
                                         hipStream_t stream);

/* ---- sparse latent attention ---------------------------------------------
 * For every query row r and head h: keys = the selected main-KV latents
 * {x_j : j = idx[r][s] >= 0} followed by the row's SWA rows; K = V = the
 * 512-channel latent (MQA over a latent shared by all heads); one softmax over
 * all of them (report 2.3: each query attends to the selected entries together
 * with the SWA KV; the reading note's Figure 4 reading: the selected main KV is
 * concatenated with the SWA KV for core attention).
 *   out[r][h] = sum_u softmax_u(scale * q[r][h] . key_u) * key_u   (fp32)
 *   lse[r][h] = log sum_u exp(scale * q[r][h] . key_u)               (optional)
 * Main-KV values are those of csa2_gather_dequant with the same kv_fmt.
 * q_bf16: [total_q][Hm][512]; swa_rows: the SWA rows in the format and layout of `swa`;
 * out: [total_q][Hm][512] f32; lse: [total_q][Hm] f32 or NULL (all device).
 * Supported: Hm a multiple of 16, 1 <= K <= 2048, window <= 1024.
 * Workspace (optional): with csa2_workspace_size(CSA2_WS_SPARSE_ATTN, ...)
 * bytes the call may split each row's keys over several workgroups when the
 * batch is small and merge the parts; with less (or NULL) it splits less (or
 * not at all).  Results agree either way within the tolerance of a softmax
 * merge, not bit for bit. */
CSA2_API csa2_status csa2_sparse_attn(const csa2_batch* batch, int32_t Hm, const uint16_t* q_bf16, int32_t kv_fmt,
                                      const uint8_t* kv_fp4, const uint8_t* kv_sc, const int32_t* idx, int32_t K,
                                      const void* swa_rows, const csa2_swa_layout* swa, float softmax_scale,
                                      float* out, float* lse, void* ws, size_t ws_bytes, hipStream_t stream);

/* ---- sparse attention with the RoPE steps fused ---------------------------
 * The report's kernel flow fuses RoPE, attention, RoPE and a cast into one
 * kernel (section 3.2, FlashMLA's RoPE-attention-RoPE-cast).  With q_bf16 the
 * query before RoPE, this equals bit for bit
 *   csa2_rope_cast(f32(q_bf16), rope_cs, 0) -> csa2_sparse_attn ->
 *   csa2_rope_cast(out, rope_cs, 1)
 * in one pass: the query is rotated (channels 448..511 in pairs
 * (448 + 2p, 449 + 2p) by the row's angles rope_cs[row][p] = cos, sin) and cast
 * back to bf16 as it is loaded; the output's rotated channels are turned back
 * (the angle negated) and every channel is cast to bf16 to nearest even as it
 * is stored.  The log-sum-exp is that of csa2_sparse_attn.
 * q_bf16:   [total_q][Hm][512] bf16 before RoPE (device, 16-byte aligned).
 * rope_cs:  [total_q][32][2] f32 (device, 16-byte aligned).
 * out_bf16: [total_q][Hm][512] bf16 (device, 4-byte aligned).
 * The other arguments, the workspace and the supported sizes are those of
 * csa2_sparse_attn. */
CSA2_API csa2_status csa2_sparse_attn_rope(const csa2_batch* batch, int32_t Hm, const uint16_t* q_bf16,
                                           const float* rope_cs, int32_t kv_fmt, const uint8_t* kv_fp4,
                                           const uint8_t* kv_sc, const int32_t* idx, int32_t K, const void* swa_rows,
                                           const csa2_swa_layout* swa, float softmax_scale, uint16_t* out_bf16,
                                           float* lse, void* ws, size_t ws_bytes, hipStream_t stream);

/* ---- layer chain ---------------------------------------------------------
 * Runs layers in order with the modes of report 2.3.1 (the reading note's mode
 * table): FULL scores every visible entry of its own caches, takes Top-K and,
 * when flagged CSA2_LAYER_BUILD_POOL, the block pool from the same scores;
 * REINDEX scores the pool (every visible entry when no pool exists) against
 * the latest Full layer's indexer K with its own q and takes Top-K; REUSE
 * attends with the latest indices; SWA_ONLY attends to its window only.  Every
 * layer attends with its own q_main and SWA rows over the latest Full layer's
 * main KV.  Results equal the composition of the calls above bit for bit. */
typedef struct csa2_layer {
    int32_t mode;                /* CSA2_MODE_* */
    int32_t flags;               /* CSA2_LAYER_BUILD_POOL (FULL only) */
    int32_t q_fmt;               /* CSA2_Q_FP4 / CSA2_Q_FP8 / CSA2_Q_MXFP4 (FULL, REINDEX); a
                                    REINDEX layer uses CSA2_Q_MXFP4 exactly when its
                                    source Full layer does (the indexer K's scales
                                    follow the format), else CSA2_ERR_INVALID_ARG */
    int32_t kv_fmt;              /* CSA2_KV_* of kv_sc (FULL: the layers up to the next Full layer read it) */
    const void* q_idx;           /* (device) indexer q (FULL, REINDEX) */
    const uint8_t* q_sc;         /* (device) [total_q][H], or [total_q][H][4] (CSA2_Q_MXFP4) */
    const float* w;              /* (device) [total_q][H] */
    const uint8_t* kv_fp4;       /* (device) main KV of this layer (FULL) */
    const uint8_t* kv_sc;
    const uint8_t* k_fp4;        /* (device) indexer K of this layer (FULL) */
    const uint8_t* k_sc;
    const uint16_t* q_main;      /* (device) [total_q][Hm][512] bf16 */
    const void* swa;             /* (device) SWA rows of this layer, in the format and layout of the chain's swa layout */
    float* out;                  /* (device) [total_q][Hm][512] */
    float* lse;                  /* (device) [total_q][Hm] or NULL */
    int32_t* idx_out;            /* (device) [total_q][K] or NULL: the indices this layer attended with */
} csa2_layer;

typedef struct csa2_chain_params {
    int32_t H;                   /* indexer heads (32 or 64) */
    int32_t Hm;                  /* main query heads (multiple of 16) */
    int32_t K;                   /* Top-K (<= 2048) */
    int32_t block;               /* pool block size (8) */
    int32_t max_blocks;          /* pool blocks (<= 2048) */
    float softmax_scale;         /* 1/sqrt(512) for the report's latent */
    /* Optional (NULL = unused): events recorded on `stream` immediately before
     * and after the index-scan kernel of the chain's first Full layer, so that
     * a caller can time that kernel alone. */
    hipEvent_t scan_begin;
    hipEvent_t scan_end;
} csa2_chain_params;

/* pool_blocks [total_q][max_blocks], pool_pos [total_q][max_blocks*block],
 * pool_count [total_q] (device, each may be NULL): the pool, when one is built.
 * Workspace: csa2_workspace_size(CSA2_WS_LAYER_CHAIN, ...). */
CSA2_API csa2_status csa2_layer_chain(const csa2_batch* batch, const csa2_chain_params* params, int32_t n_layers,
                                      const csa2_layer* layers, const csa2_swa_layout* swa, int32_t* pool_blocks,
                                      int32_t* pool_pos, int32_t* pool_count, void* ws, size_t ws_bytes,
                                      hipStream_t stream);

/* ---- workspace, status ----------------------------------------------------- */
#define CSA2_WS_TOPK 1
#define CSA2_WS_BLOCK_POOL 2
#define CSA2_WS_SPARSE_ATTN 3
#define CSA2_WS_LAYER_CHAIN 4

/* Bytes of workspace the call `which` needs for this batch; K and max_blocks
 * as the call will be made (ignored where irrelevant); n_layers for the chain.
 * Returns 0 on invalid arguments. */
CSA2_API size_t csa2_workspace_size(int32_t which, const csa2_batch* batch, int32_t K, int32_t max_blocks,
                                    int32_t n_layers);

CSA2_API const char* csa2_status_string(csa2_status s);
/* The hipError_t of the last CSA2_ERR_HIP returned on this host thread. */
CSA2_API int32_t csa2_last_hip_error(void);
CSA2_API int32_t csa2_version(void);

#ifdef __cplusplus
}
#endif
#endif /* CSA2_H */
