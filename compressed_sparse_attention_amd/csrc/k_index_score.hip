// Lightning-indexer scoring on gfx950 matrix cores.
//
// score(r, j) = 2^(k_sc[j]-127) * sum_h w[r,h] * ReLU(d_h * 2^(q_sc[r,h]-127)),
// d_h = q[r,h,:] . k[j,:] over the 128 indexer channels (report "DeepSeek-V4.1-
// Flash: Pushing the Limits of KV Cache Compression", section 2.3: the indexer
// scores main-KV entries with indexer Q and indexer K; section 2.3.1: Full mode
// scores every visible entry, Reindex mode rescores the shared indexer K).
//
// The per-head dot products run as one dense contraction per 64-position tile:
// D[head][position] = Q[head][128] x K[position][128]^T on v_mfma_scale_f32_
// 32x32x64_f8f6f4 (E2M1 or E4M3 A operand, E2M1 B operand, the query row's E8M0
// scale applied by the instruction).  Every product is exact and every partial
// sum is a multiple of 2^-2 (FP4 x FP4) or 2^-10 (FP8 x FP4) below 2^24 units, so
// D is exact whatever the accumulation order.  The head sum is then evaluated
// per position in one lane, in the fixed order h = 0..H-1 with one fused
// multiply-add per head, so the binary32 score is reproducible bit for bit.
//
// MFMA layouts (32x32x64, measured on gfx950): lane l supplies A row l%32 and
// B column l%32; for E2M1 operands lane half g = l/32 supplies k = 32g + e for
// nibble e = 0..31 of its 16 bytes (low nibble first); for E4M3 operands byte e
// of the 32 supplies k = 16g + e (e < 16) and k = 32 + 16g + (e-16) (e >= 16).
// Result element (row m, column n) lands in lane n + 32*((m/4)%2), register
// 4*(m/8) + m%4.
#include "csa2_internal.h"

namespace csa2 {
namespace {

__device__ __forceinline__ v16f mfma_scaled(const v8i& a, const v8i& b, const v16f& c, int sa, int fmt_a) {
    if (fmt_a == 0)  // E4M3 A, E2M1 B
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 4, 0, sa, 0, 127);
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 4, 4, 0, sa, 0, 127);
}

__device__ __forceinline__ v8i widen(v4i x) { return v8i{x[0], x[1], x[2], x[3], 0, 0, 0, 0}; }

__device__ __forceinline__ v4i ld16(const uint8_t* p) { return *reinterpret_cast<const v4i*>(p); }

// After the MFMAs of one 64-position tile, acc[mt][nt] holds heads 32mt.. of
// positions 32nt + l%32.  Swap the upper half of nt = 0 with the lower half of
// nt = 1 so that every lane holds all H heads of position p0 + lane, then run
// the canonical head sum.  `w` points at the row's H weights (uniform).
// Callers run it with all 64 lanes active (the swap reads the partner lane)
// and predicate only the store.
template <int NMT>
__device__ __forceinline__ float head_sum(v16f (&acc)[NMT][2], const float* __restrict__ w) {
    float x[NMT][16], y[NMT][16];
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            // element values go through __float_as_uint: a bit cast applied to a
            // vector element expression would read element 0 of the vector
            const float e0 = acc[mt][0][v], e1 = acc[mt][1][v];
            auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(e0), __float_as_uint(e1), false, false);
            x[mt][v] = __uint_as_float((unsigned)r[0]);  // rows 8*(v/4) + v%4
            y[mt][v] = __uint_as_float((unsigned)r[1]);  // rows 8*(v/4) + 4 + v%4
        }
    float s = 0.0f;
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
#pragma unroll
            for (int i = 0; i < 4; ++i) s = __builtin_fmaf(w[32 * mt + 8 * gq + i], fmaxf(x[mt][4 * gq + i], 0.0f), s);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                s = __builtin_fmaf(w[32 * mt + 8 * gq + 4 + i], fmaxf(y[mt][4 * gq + i], 0.0f), s);
        }
    return s;
}

// Histogram of the written scores over bits 30..19 (the bins the Top-K pass
// starts from), kept in LDS per query row and flushed with one global atomic
// per non-empty bin.  Negative scores (only possible with negative head
// weights) count in bin 0, as the Top-K pass orders them.
__device__ __forceinline__ uint32_t score_bin(float s) {
    const uint32_t u = __float_as_uint(s);
    return (u & 0x80000000u) ? 0u : (u >> 19);
}

__device__ __forceinline__ void hist_clear(uint32_t* h, int nbins) {
    for (int i = threadIdx.x; i < nbins; i += blockDim.x) h[i] = 0;
}

__device__ __forceinline__ void hist_flush(const uint32_t* h, uint32_t* __restrict__ g) {
    for (int i = threadIdx.x; i < kHistBins; i += blockDim.x)
        if (h[i]) atomicAdd(&g[i], h[i]);
}

// ---------------------------------------------------------------------------
// Decode scan: every sequence has at most TQ query rows (1 for plain decode, 4
// for the speculative-verify shape); they share one pass over the sequence's
// indexer K.  Grid (chunks, n_seq); 4 waves; each wave takes 64-position tiles.
// FP4 x FP4; channel c of a row sits at (lane half g, k-step ks, nibble e)
// with c = 64g + 32ks + e for both operands.
// ---------------------------------------------------------------------------
template <int H, int TQ, bool HIST>
__global__ __launch_bounds__(256) void k_score_decode(const uint8_t* __restrict__ q, const uint8_t* __restrict__ q_sc,
                                                      const float* __restrict__ w, const uint8_t* __restrict__ k,
                                                      const uint8_t* __restrict__ k_sc,
                                                      const int64_t* __restrict__ entry_off,
                                                      const int32_t* __restrict__ q_off,
                                                      const int32_t* __restrict__ q_pos, int ratio,
                                                      float* __restrict__ scores, int64_t stride, int chunk,
                                                      uint32_t* __restrict__ hist) {
    constexpr int NMT = H / 32;
    __shared__ uint32_t hl[HIST ? TQ * kHistBins : 1];
    const int b = blockIdx.y;
    const int64_t e0 = entry_off[b];
    const int64_t n = entry_off[b + 1] - e0;
    const int64_t c0 = (int64_t)blockIdx.x * chunk;
    if (c0 >= n) return;
    const int64_t c1 = c0 + chunk < n ? c0 + chunk : n;
    const int r0 = q_off[b];
    const int nq = q_off[b + 1] - r0;
    if (nq <= 0) return;  // a sequence without query rows has no scores
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 5, li = lane & 31;
    if (HIST) hist_clear(hl, TQ * kHistBins);

    v8i A[TQ][NMT][2];
    int SA[TQ][NMT];
    int64_t vis[TQ];
#pragma unroll
    for (int t = 0; t < TQ; ++t) {
        const int row = r0 + (t < nq ? t : 0);
        vis[t] = visible_count(n, q_pos[row], ratio);
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt) {
            const uint8_t* qr = q + ((int64_t)row * H + 32 * mt + li) * 64 + 32 * g;
            A[t][mt][0] = widen(ld16(qr));
            A[t][mt][1] = widen(ld16(qr + 16));
            SA[t][mt] = q_sc[(int64_t)row * H + 32 * mt + li];
        }
    }
    if (HIST) __syncthreads();

    // software pipeline: the indexer K of the next tile is in flight while
    // the current tile computes
    v4i Bn[2][2];
    int ekn = 127;
    auto fetch = [&](int64_t p0) {
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            int64_t j = p0 + 32 * nt + li;
            j = j < n ? j : n - 1;
            const uint8_t* kr = k + (e0 + j) * 64 + 32 * g;
            Bn[nt][0] = ld16(kr);
            Bn[nt][1] = ld16(kr + 16);
        }
        const int64_t jl = p0 + lane;
        ekn = jl < n ? (int)k_sc[e0 + jl] : 127;
    };
    int64_t p0 = c0 + 64 * wave;
    if (p0 < c1) fetch(p0);
    for (; p0 < c1; p0 += 256) {
        v8i B[2][2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) B[nt][ks] = widen(Bn[nt][ks]);
        const int ek = ekn;
        if (p0 + 256 < c1) fetch(p0 + 256);
        const int64_t jl = p0 + lane;
#pragma unroll
        for (int t = 0; t < TQ; ++t) {
            if (t >= nq) break;
            v16f acc[NMT][2];
#pragma unroll
            for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    acc[mt][nt] = v16f{};
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks) acc[mt][nt] = mfma_scaled(A[t][mt][ks], B[nt][ks], acc[mt][nt], SA[t][mt], 4);
                }
            const float s = head_sum<NMT>(acc, w + (int64_t)(r0 + t) * H);
            if (jl < n) {
                const bool visible = jl < vis[t];
                const float sc = visible ? ldexpf(s, ek - 127) : -INFINITY;
                scores[(int64_t)(r0 + t) * stride + jl] = sc;
                if (HIST && visible) atomicAdd(&hl[t * kHistBins + score_bin(sc)], 1u);
            }
        }
    }
    if (HIST) {
        __syncthreads();
        for (int t = 0; t < TQ && t < nq; ++t) hist_flush(hl + t * kHistBins, hist + (int64_t)(r0 + t) * kHistBins);
    }
}

// ---------------------------------------------------------------------------
// Candidate (Reindex) scoring: slot s of row r scores entry cand[r][s].
// Grid (slot chunks of 1024, total_q).  Same operand mapping as the decode scan.
// ---------------------------------------------------------------------------
template <int H, bool HIST>
__global__ __launch_bounds__(256) void k_score_cand(const uint8_t* __restrict__ q, const uint8_t* __restrict__ q_sc,
                                                    const float* __restrict__ w, const uint8_t* __restrict__ k,
                                                    const uint8_t* __restrict__ k_sc,
                                                    const int64_t* __restrict__ entry_off,
                                                    const int32_t* __restrict__ row_seq,
                                                    const int32_t* __restrict__ q_pos, int ratio,
                                                    const int32_t* __restrict__ cand, int cand_stride,
                                                    float* __restrict__ scores, int64_t stride,
                                                    uint32_t* __restrict__ hist) {
    constexpr int NMT = H / 32;
    constexpr int CH = 1024;
    __shared__ uint32_t hl[HIST ? kHistBins : 1];
    const int row = blockIdx.y;
    const int s0 = blockIdx.x * CH;
    if (s0 >= cand_stride) return;
    const int s1 = s0 + CH < cand_stride ? s0 + CH : cand_stride;
    const int b = row_seq[row];
    const int64_t e0 = entry_off[b];
    const int64_t n = entry_off[b + 1] - e0;
    const int64_t vis = visible_count(n, q_pos[row], ratio);
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 5, li = lane & 31;
    const int32_t* crow = cand + (int64_t)row * cand_stride;
    float* srow = scores + (int64_t)row * stride;
    if (vis <= 0) {
        for (int s = s0 + threadIdx.x; s < s1; s += 256) srow[s] = -INFINITY;
        return;
    }
    if (HIST) hist_clear(hl, kHistBins);
    v8i A[NMT][2];
    int SA[NMT];
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
        const uint8_t* qr = q + ((int64_t)row * H + 32 * mt + li) * 64 + 32 * g;
        A[mt][0] = widen(ld16(qr));
        A[mt][1] = widen(ld16(qr + 16));
        SA[mt] = q_sc[(int64_t)row * H + 32 * mt + li];
    }
    if (HIST) __syncthreads();
    for (int p0 = s0 + 64 * wave; p0 < s1; p0 += 256) {
        v8i B[2][2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const int s = p0 + 32 * nt + li;
            int64_t j = s < s1 ? (int64_t)crow[s] : -1;
            j = (j >= 0 && j < vis) ? j : 0;
            const uint8_t* kr = k + (e0 + j) * 64 + 32 * g;
            B[nt][0] = widen(ld16(kr));
            B[nt][1] = widen(ld16(kr + 16));
        }
        const int sl = p0 + lane;
        const int64_t jl = sl < s1 ? (int64_t)crow[sl] : -1;
        const bool ok = jl >= 0 && jl < vis;
        const int ek = ok ? (int)k_sc[e0 + jl] : 127;
        v16f acc[NMT][2];
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                acc[mt][nt] = v16f{};
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) acc[mt][nt] = mfma_scaled(A[mt][ks], B[nt][ks], acc[mt][nt], SA[mt], 4);
            }
        const float sc = head_sum<NMT>(acc, w + (int64_t)row * H);
        if (sl < s1) {
            const float v = ok ? ldexpf(sc, ek - 127) : -INFINITY;
            srow[sl] = v;
            // the Top-K pass over a candidate list takes its first cand_count
            // slots, which are the non-empty ones of a pool list
            if (HIST && ok) atomicAdd(&hl[score_bin(v)], 1u);
        }
    }
    if (HIST) {
        __syncthreads();
        hist_flush(hl, hist + (int64_t)row * kHistBins);
    }
}

// ---------------------------------------------------------------------------
// Prefill scoring: many query rows per sequence.  Grid (position tiles of PT,
// query groups of 8 rows, n_seq).  The tile's indexer K is staged in LDS once
// and each wave keeps two query rows in registers.  Channel c of a row sits at
// k-step ks = c/64, k = c%64 for both operands (the E4M3 layout fixes it for A;
// B is loaded to match).
// ---------------------------------------------------------------------------
template <int H, int QFMT>
__global__ __launch_bounds__(256) void k_score_prefill(const uint8_t* __restrict__ q,
                                                       const uint8_t* __restrict__ q_sc,
                                                       const float* __restrict__ w, const uint8_t* __restrict__ k,
                                                       const uint8_t* __restrict__ k_sc,
                                                       const int64_t* __restrict__ entry_off,
                                                       const int32_t* __restrict__ q_off,
                                                       const int32_t* __restrict__ q_pos, int ratio,
                                                       float* __restrict__ scores, int64_t stride) {
    constexpr int NMT = H / 32;
    constexpr int PT = 1024;
    constexpr int QG = 8;
    constexpr int QROW = QFMT == 0 ? 128 : 64;  // bytes per head row
    __shared__ __attribute__((aligned(16))) uint8_t ks_lds[PT * 64];
    __shared__ uint8_t ksc_lds[PT];
    const int b = blockIdx.z;
    const int64_t e0 = entry_off[b];
    const int64_t n = entry_off[b + 1] - e0;
    const int rb = q_off[b], nrow_b = q_off[b + 1] - rb;
    const int r0 = rb + QG * blockIdx.y;
    if (QG * (int)blockIdx.y >= nrow_b) return;
    const int nr = nrow_b - QG * (int)blockIdx.y < QG ? nrow_b - QG * (int)blockIdx.y : QG;
    // rows are in increasing token order within a sequence only by convention;
    // take the largest visibility of the group to bound the tile range
    int64_t vmax = 0;
    for (int i = 0; i < nr; ++i) {
        const int64_t v = visible_count(n, q_pos[r0 + i], ratio);
        vmax = v > vmax ? v : vmax;
    }
    const int64_t p_base = (int64_t)blockIdx.x * PT;
    if (p_base >= vmax) {
        // nothing visible here: the rows' slots in this tile are -inf
        for (int i = 0; i < nr; ++i)
            for (int64_t j = p_base + threadIdx.x; j < p_base + PT && j < n; j += 256)
                scores[(int64_t)(r0 + i) * stride + j] = -INFINITY;
        return;
    }
    const int64_t p_end = p_base + PT < n ? p_base + PT : n;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 5, li = lane & 31;

    // stage the tile's indexer K (rows past the sequence end are clamped)
    for (int i = threadIdx.x; i < PT * 4; i += 256) {
        const int row = i >> 2, part = i & 3;
        int64_t j = p_base + row;
        j = j < n ? j : n - 1;
        *reinterpret_cast<v4i*>(ks_lds + row * 64 + part * 16) = ld16(k + (e0 + j) * 64 + part * 16);
    }
    for (int i = threadIdx.x; i < PT; i += 256) {
        const int64_t j = p_base + i;
        ksc_lds[i] = j < n ? k_sc[e0 + j] : 127;
    }

    // two query rows per wave, in registers
    v8i A[2][NMT][2];
    int SA[2][NMT];
    int64_t vis[2];
    int rows[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int qi = 2 * wave + u;
        rows[u] = qi < nr ? r0 + qi : -1;
        const int row = qi < nr ? r0 + qi : r0;
        vis[u] = visible_count(n, q_pos[row], ratio);
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt) {
            const uint8_t* qr = q + ((int64_t)row * H + 32 * mt + li) * QROW;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                if (QFMT == 0) {
                    const v4i lo = ld16(qr + 64 * ks + 16 * g);
                    const v4i hi = ld16(qr + 64 * ks + 32 + 16 * g);
                    A[u][mt][ks] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                } else {
                    A[u][mt][ks] = widen(ld16(qr + 32 * ks + 16 * g));
                }
            }
            SA[u][mt] = q_sc[(int64_t)row * H + 32 * mt + li];
        }
    }
    __syncthreads();

    for (int tile = 0; tile < PT / 64; ++tile) {
        const int64_t p0 = p_base + 64 * tile;
        if (p0 >= p_end) break;
        v8i B[2][2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                B[nt][ks] = widen(*reinterpret_cast<const v4i*>(ks_lds + (64 * tile + 32 * nt + li) * 64 + 32 * ks + 16 * g));
        const int64_t jl = p0 + lane;
        const int ek = ksc_lds[64 * tile + lane];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            if (rows[u] < 0) break;
            if (p0 >= vis[u]) {
                if (jl < n) scores[(int64_t)rows[u] * stride + jl] = -INFINITY;
                continue;
            }
            v16f acc[NMT][2];
#pragma unroll
            for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    acc[mt][nt] = v16f{};
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks)
                        acc[mt][nt] = mfma_scaled(A[u][mt][ks], B[nt][ks], acc[mt][nt], SA[u][mt], QFMT == 0 ? 0 : 4);
                }
            const float s = head_sum<NMT>(acc, w + (int64_t)rows[u] * H);
            if (jl < n) scores[(int64_t)rows[u] * stride + jl] = jl < vis[u] ? ldexpf(s, ek - 127) : -INFINITY;
        }
    }
}

// ---------------------------------------------------------------------------
// Prefill scoring with E4M3 queries.  gfx950's E4M3 x E2M1 MFMA keeps only a
// window of about 14 bits below its largest product when it sums a block of
// products (measured: 2^5 + 2^-9 comes back as 2^5), while these dot products
// span up to 16 bits (|q| < 16 on a 2^-9 grid, |k| <= 6 on a 2^-1 grid).  Both
// operands are exact in bf16, and v_mfma_f32_32x32x16_bf16 sums them exactly
// (measured up to a 23-bit window), so this kernel converts both to bf16
// (the query row's E8M0 scale folded into the conversion, which is exact) and
// contracts on the bf16 matrix cores.  Channel c of a row sits at k-step
// ks = c/16, lane half g = (c/8)%2, element c%8.  Grid and staging as in
// k_score_prefill; two query rows per wave.
// ---------------------------------------------------------------------------
template <int H>
__global__ __launch_bounds__(256) void k_score_prefill_fp8(const uint8_t* __restrict__ q,
                                                           const uint8_t* __restrict__ q_sc,
                                                           const float* __restrict__ w,
                                                           const uint8_t* __restrict__ k,
                                                           const uint8_t* __restrict__ k_sc,
                                                           const int64_t* __restrict__ entry_off,
                                                           const int32_t* __restrict__ q_off,
                                                           const int32_t* __restrict__ q_pos, int ratio,
                                                           float* __restrict__ scores, int64_t stride) {
    constexpr int NMT = H / 32;
    constexpr int PT = 1024;
    constexpr int QG = 8;
    __shared__ __attribute__((aligned(16))) uint8_t ks_lds[PT * 64];
    __shared__ uint8_t ksc_lds[PT];
    const int b = blockIdx.z;
    const int64_t e0 = entry_off[b];
    const int64_t n = entry_off[b + 1] - e0;
    const int rb = q_off[b], nrow_b = q_off[b + 1] - rb;
    const int r0 = rb + QG * blockIdx.y;
    if (QG * (int)blockIdx.y >= nrow_b) return;
    const int nr = nrow_b - QG * (int)blockIdx.y < QG ? nrow_b - QG * (int)blockIdx.y : QG;
    int64_t vmax = 0;
    for (int i = 0; i < nr; ++i) {
        const int64_t v = visible_count(n, q_pos[r0 + i], ratio);
        vmax = v > vmax ? v : vmax;
    }
    const int64_t p_base = (int64_t)blockIdx.x * PT;
    if (p_base >= vmax) {
        for (int i = 0; i < nr; ++i)
            for (int64_t j = p_base + threadIdx.x; j < p_base + PT && j < n; j += 256)
                scores[(int64_t)(r0 + i) * stride + j] = -INFINITY;
        return;
    }
    const int64_t p_end = p_base + PT < n ? p_base + PT : n;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 5, li = lane & 31;

    for (int i = threadIdx.x; i < PT * 4; i += 256) {
        const int row = i >> 2, part = i & 3;
        int64_t j = p_base + row;
        j = j < n ? j : n - 1;
        *reinterpret_cast<v4i*>(ks_lds + row * 64 + part * 16) = ld16(k + (e0 + j) * 64 + part * 16);
    }
    for (int i = threadIdx.x; i < PT; i += 256) {
        const int64_t j = p_base + i;
        ksc_lds[i] = j < n ? k_sc[e0 + j] : 127;
    }

    v8bf A[2][NMT][8];
    int64_t vis[2];
    int rows[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int qi = 2 * wave + u;
        rows[u] = qi < nr ? r0 + qi : -1;
        const int row = qi < nr ? r0 + qi : r0;
        vis[u] = visible_count(n, q_pos[row], ratio);
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt) {
            const uint8_t* qr = q + ((int64_t)row * H + 32 * mt + li) * 128 + 8 * g;
            const float sc = __builtin_ldexpf(1.0f, (int)q_sc[(int64_t)row * H + 32 * mt + li] - 127);
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                const uint2 c = *reinterpret_cast<const uint2*>(qr + 16 * ks);
                auto lo0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.x, sc, false);
                auto lo1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.x, sc, true);
                auto hi0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.y, sc, false);
                auto hi1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.y, sc, true);
                A[u][mt][ks] = v8bf{lo0[0], lo0[1], lo1[0], lo1[1], hi0[0], hi0[1], hi1[0], hi1[1]};
            }
        }
    }
    __syncthreads();

    for (int tile = 0; tile < PT / 64; ++tile) {
        const int64_t p0 = p_base + 64 * tile;
        if (p0 >= p_end) break;
        const int64_t jl = p0 + lane;
        const int ek = ksc_lds[64 * tile + lane];
        v16f acc[2][NMT][2];
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) acc[u][mt][nt] = v16f{};
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                // position 64 tile + 32 nt + li, channels 16 ks + 8 g .. +8 = FP4 bytes 8 ks + 4 g .. +4
                const uint32_t c =
                    *reinterpret_cast<const uint32_t*>(ks_lds + (64 * tile + 32 * nt + li) * 64 + 8 * ks + 4 * g);
                auto b0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, 1.0f, 0);
                auto b1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, 1.0f, 1);
                auto b2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, 1.0f, 2);
                auto b3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, 1.0f, 3);
                const v8bf B = {b0[0], b0[1], b1[0], b1[1], b2[0], b2[1], b3[0], b3[1]};
#pragma unroll
                for (int u = 0; u < 2; ++u)
#pragma unroll
                    for (int mt = 0; mt < NMT; ++mt)
                        acc[u][mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[u][mt][ks], B, acc[u][mt][nt], 0, 0, 0);
            }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            if (rows[u] < 0) break;  // wave-uniform
            float* dst = scores + (int64_t)rows[u] * stride + jl;
            if (p0 >= vis[u]) {  // wave-uniform
                if (jl < n) *dst = -INFINITY;
                continue;
            }
            // all 64 lanes must run the head sum: its permlane32_swap reads the partner lane
            const float s = head_sum<NMT>(acc[u], w + (int64_t)rows[u] * H);
            if (jl < n) *dst = jl < vis[u] ? ldexpf(s, ek - 127) : -INFINITY;
        }
    }
}

}  // namespace

hipError_t launch_index_score(const ScoreLaunch& a, hipStream_t s) {
    const csa2_batch* b = a.b;
    if (a.cand) {
        dim3 grid((a.cand_stride + 1023) / 1024, a.g.total_q);
#define CSA2_CAND(HH, HI)                                                                                        \
    hipLaunchKernelGGL((k_score_cand<HH, HI>), grid, dim3(256), 0, s, a.q, a.q_sc, a.w, a.k, a.k_sc,            \
                       b->d_entry_off, b->d_row_seq, b->d_q_pos, b->ratio, a.cand, a.cand_stride, a.scores,      \
                       a.stride, a.hist)
        if (a.H == 64) {
            if (a.hist) CSA2_CAND(64, true); else CSA2_CAND(64, false);
        } else {
            if (a.hist) CSA2_CAND(32, true); else CSA2_CAND(32, false);
        }
#undef CSA2_CAND
        return hipGetLastError();
    }
    if (a.q_fmt == CSA2_Q_FP4 && a.g.max_q_per_seq <= 4) {
        const int chunk = 4096;
        dim3 grid((unsigned)((a.g.max_entries + chunk - 1) / chunk), a.g.n_seq);
#define CSA2_DEC(HH, TT, HI)                                                                                     \
    hipLaunchKernelGGL((k_score_decode<HH, TT, HI>), grid, dim3(256), 0, s, a.q, a.q_sc, a.w, a.k, a.k_sc,      \
                       b->d_entry_off, b->d_q_off, b->d_q_pos, b->ratio, a.scores, a.stride, chunk, a.hist)
        const bool one = a.g.max_q_per_seq <= 1;
        if (a.H == 64) {
            if (a.hist) { if (one) CSA2_DEC(64, 1, true); else CSA2_DEC(64, 4, true); }
            else { if (one) CSA2_DEC(64, 1, false); else CSA2_DEC(64, 4, false); }
        } else {
            if (a.hist) { if (one) CSA2_DEC(32, 1, true); else CSA2_DEC(32, 4, true); }
            else { if (one) CSA2_DEC(32, 1, false); else CSA2_DEC(32, 4, false); }
        }
#undef CSA2_DEC
        return hipGetLastError();
    }
    dim3 grid((unsigned)((a.g.max_entries + 1023) / 1024), (unsigned)((a.g.max_q_per_seq + 7) / 8), a.g.n_seq);
#define CSA2_PRE(HH, FF)                                                                                          \
    hipLaunchKernelGGL((k_score_prefill<HH, FF>), grid, dim3(256), 0, s, a.q, a.q_sc, a.w, a.k, a.k_sc,          \
                       b->d_entry_off, b->d_q_off, b->d_q_pos, b->ratio, a.scores, a.stride)
    if (a.q_fmt == CSA2_Q_FP8) {
        if (a.H == 64)
            hipLaunchKernelGGL((k_score_prefill_fp8<64>), grid, dim3(256), 0, s, a.q, a.q_sc, a.w, a.k, a.k_sc,
                               b->d_entry_off, b->d_q_off, b->d_q_pos, b->ratio, a.scores, a.stride);
        else
            hipLaunchKernelGGL((k_score_prefill_fp8<32>), grid, dim3(256), 0, s, a.q, a.q_sc, a.w, a.k, a.k_sc,
                               b->d_entry_off, b->d_q_off, b->d_q_pos, b->ratio, a.scores, a.stride);
    } else {
        if (a.H == 64) CSA2_PRE(64, 4); else CSA2_PRE(32, 4);
    }
#undef CSA2_PRE
    return hipGetLastError();
}

}  // namespace csa2
