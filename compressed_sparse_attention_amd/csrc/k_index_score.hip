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
// The report's indexer format (section 2.4.4: FP4 indexer queries and keys in
// OCP MXFP4) carries one E8M0 per 32 channels on both sides.  With it (MX) the
// instruction applies the query's block scale (A) and the key's (B) per lane
// half, so D already holds the scaled dot product and no per-entry factor
// follows the head sum.  The blocks of a q/K pair then sit on grids up to
// 2^spread apart; with the spreads of MX-quantised rows (a few powers of two)
// every partial sum still fits the exact range, which the parity tests check.
//
// MFMA layouts (32x32x64, measured on gfx950): lane l supplies A row l%32 and
// B column l%32; for E2M1 operands lane half g = l/32 supplies k = 32g + e for
// nibble e = 0..31 of its 16 bytes (low nibble first); for E4M3 operands byte e
// of the 32 supplies k = 16g + e (e < 16) and k = 32 + 16g + (e-16) (e >= 16).
// Result element (row m, column n) lands in lane n + 32*((m/4)%2), register
// 4*(m/8) + m%4.
#include <hip/hip_ext.h>

#include "csa2_internal.h"

namespace csa2 {
namespace {

__device__ __forceinline__ v16f mfma_scaled(const v8i& a, const v8i& b, const v16f& c, int sa, int fmt_a) {
    if (fmt_a == 0)  // E4M3 A, E2M1 B
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 4, 0, sa, 0, 127);
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 4, 4, 0, sa, 0, 127);
}

// FP4 x FP4 with an E8M0 per lane for each operand (bits 7..0 of sa and sb)
__device__ __forceinline__ v16f mfma_fp4_mx(const v8i& a, const v8i& b, const v16f& c, int sa, int sb) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 4, 4, 0, sa, 0, sb);
}

// byte i of a packed word of four E8M0 scales
__device__ __forceinline__ int scale_byte(uint32_t w, int i) { return (int)((w >> (8 * i)) & 255u); }

// E2M1 operands occupy the low four dwords of the 8-dword operand; the upper
// four are never read, so they are left undefined (no registers zeroed)
__device__ __forceinline__ v8i widen(v4i x) { return __builtin_shufflevector(x, x, 0, 1, 2, 3, -1, -1, -1, -1); }

__device__ __forceinline__ v4i ld16(const uint8_t* p) { return *reinterpret_cast<const v4i*>(p); }

// max(x, 0) as one integer max on the bit pattern: negative floats (and -0)
// are negative integers and map to +0, the rest are unchanged.  fmaxf would
// add a NaN-quieting max in front of it; the MFMA results are never NaN.
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// Maxima across lanes with DPP moves (VALU operands, no LDS round trip):
// max8 leaves the maximum of each group of 8 lanes in all 8 of them; from
// there, max32_8 leaves the maximum of each 32-lane half in its lane 31 (and
// 63) and max64_8 the maximum of the wave in lane 63 (other lanes hold
// partial maxima).
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ float dpp_max(float v) {
    return fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, ROWS, 0xF,
                                                               false)));
}
__device__ __forceinline__ float max8(float v) {
    v = dpp_max<0xB1>(v);          // quad_perm 1,0,3,2: lanes xor 1
    v = dpp_max<0x4E>(v);          // quad_perm 2,3,0,1: lanes xor 2
    return dpp_max<0x141>(v);      // row_half_mirror: the two quads of each 8 lanes
}
__device__ __forceinline__ float max32_8(float v) {
    v = dpp_max<0x140>(v);          // row_mirror: the two 8-lane halves of each 16-lane row
    return dpp_max<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3: lane 15 of the row below
}
__device__ __forceinline__ float max64_8(float v) {
    return dpp_max<0x143, 0xC>(max32_8(v));  // row_bcast:31 into rows 2 and 3: lane 31
}

// After the MFMAs of one 64-position tile, acc[nt] holds 32 heads of
// positions 32nt + l%32.  Swap the upper half of nt = 0 with the lower half of
// nt = 1 so that every lane holds the 32 heads of position p0 + lane, then
// continue the canonical head sum over them from s.  `w` points at the 32
// weights of these heads (uniform).  Callers run it with all 64 lanes active
// (the swap reads the partner lane) and predicate only the store.
__device__ __forceinline__ float head_sum_32(v16f (&acc)[2], const float* __restrict__ w, float s) {
    float x[16], y[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        // element values go through __float_as_uint: a bit cast applied to a
        // vector element expression would read element 0 of the vector
        const float e0 = acc[0][v], e1 = acc[1][v];
        auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(e0), __float_as_uint(e1), false, false);
        x[v] = __uint_as_float((unsigned)r[0]);  // heads 8*(v/4) + v%4
        y[v] = __uint_as_float((unsigned)r[1]);  // heads 8*(v/4) + 4 + v%4
    }
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
#pragma unroll
        for (int i = 0; i < 4; ++i) s = __builtin_fmaf(w[8 * gq + i], relu(x[4 * gq + i]), s);
#pragma unroll
        for (int i = 0; i < 4; ++i) s = __builtin_fmaf(w[8 * gq + 4 + i], relu(y[4 * gq + i]), s);
    }
    return s;
}

// The whole head sum from +0 over NMT groups of 32 heads, h = 0 .. 32 NMT - 1.
template <int NMT>
__device__ __forceinline__ float head_sum(v16f (&acc)[NMT][2], const float* __restrict__ w) {
    float s = 0.0f;
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) s = head_sum_32(acc[mt], w + 32 * mt, s);
    return s;
}

// Histogram of the written scores over bits 30..19 (the bins the Top-K pass
// starts from), kept in LDS per query row and flushed with one global atomic
// per non-empty bin.  Negative scores (only possible with negative head
// weights) count in bin 0, where the Top-K pass selects among them by value:
// the same bin as key_bin(score_key(s)), in two operations.
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

// The decode scan counts at most 4096 positions per row, so its LDS histogram
// packs two 16-bit counts per word (bin 2i in the low half of word i).
__device__ __forceinline__ void hist16_add(uint32_t* h, uint32_t bin) { atomicAdd(&h[bin >> 1], 1u << (16 * (bin & 1))); }

// Adds the counts of bins lo .. kHistBins-1 to the global histogram g.
__device__ __forceinline__ void hist16_flush(const uint32_t* h, uint32_t* __restrict__ g, uint32_t lo = 0) {
    for (int i = threadIdx.x + (int)(lo >> 1); i < kHistBins / 2; i += blockDim.x) {
        const uint32_t v = h[i];
        if ((v & 0xFFFFu) && (uint32_t)(2 * i) >= lo) atomicAdd(&g[2 * i], v & 0xFFFFu);
        if (v >> 16) atomicAdd(&g[2 * i + 1], v >> 16);
    }
}

// ---------------------------------------------------------------------------
// Decode scan: every sequence has at most TQ query rows (1 for plain decode, 4
// for the speculative-verify shape); they share one pass over the sequence's
// indexer K.  Grid (chunks, n_seq); 4 waves; each wave takes 64-position tiles.
// FP4 x FP4; channel c of a row sits at (lane half g, k-step ks, nibble e)
// with c = 64g + 32ks + e for both operands.
//
// Outputs (OUT): kOutScores writes the score rows; kOutHist also builds the
// rows' bin histograms; kOutLocal keeps the chunk's scores in LDS and writes,
// besides the histograms, the chunk's candidate list per row (LocalOut) and,
// when asked, the block maxima of the block pool.
// ---------------------------------------------------------------------------
enum : int { kOutScores = 0, kOutHist = 1, kOutLocal = 2 };

template <int H, int TQ, int OUT, bool MX>
__global__ __launch_bounds__(256) void k_score_decode(const uint8_t* __restrict__ q, const uint8_t* __restrict__ q_sc,
                                                      const float* __restrict__ w, const uint8_t* __restrict__ k,
                                                      const uint8_t* __restrict__ k_sc,
                                                      const int64_t* __restrict__ entry_off,
                                                      const int32_t* __restrict__ q_off,
                                                      const int32_t* __restrict__ q_pos, int ratio,
                                                      float* __restrict__ scores, int64_t stride,
                                                      uint32_t* __restrict__ hist, LocalOut lo) {
    constexpr int NMT = H / 32;
    constexpr bool HIST = OUT != kOutScores;
    constexpr bool LOCAL = OUT == kOutLocal;
    constexpr int chunk = decode_chunk(TQ, LOCAL);
    __shared__ uint32_t hl[HIST ? TQ * kHistBins / 2 : 1];
    __shared__ __attribute__((aligned(16))) float sl[LOCAL ? TQ : 1][LOCAL ? chunk : 1];  // the chunk's scores per row
    __shared__ uint8_t ekl[MX ? 1 : chunk];                  // the chunk's indexer K scales (one per row)
    __shared__ float wl[TQ == 4 ? 4 * H : 1];               // the rows' head weights (four-row scan)
    __shared__ uint32_t wtot[4], found[4];
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
    if (HIST) {  // before any load is in flight: the barrier costs nothing here
        hist_clear(hl, TQ * kHistBins / 2);
        __syncthreads();
    }
    // four rows: thread i < 4H holds weight i % H of row i / H until it is
    // staged in LDS with the scales below; vis_pr[pr] is the visible count of
    // this lane's row of pair pr (row 2 pr + lane half)
    float w_own = 0.0f;
    int64_t vis_pr[2] = {0, 0};
    if constexpr (TQ == 4) {
        const int i = threadIdx.x;
        if (i < 4 * H && i / H < nq) w_own = w[(int64_t)(r0 + i / H) * H + i % H];
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) {
            const int qq = 2 * pr + g;
            vis_pr[pr] = visible_count(n, q_pos[r0 + (qq < nq ? qq : 0)], ratio);
        }
    }
    // the scales of this wave's positions (position p_w + 256 j + lane), staged
    // in LDS below once the query operands and the first two tiles are in
    // flight as well; only this wave reads them, so no barrier is needed
    const int64_t p_w = c0 + 64 * wave;
    uint8_t sb[chunk / 256];
    if constexpr (!MX) {
#pragma unroll
        for (int j = 0; j < chunk / 256; ++j) {
            const int64_t p = p_w + 256 * j + lane;
            sb[j] = p < c1 ? k_sc[e0 + p] : 0;
        }
    }

    v8i A[TQ][NMT][2];
    // the query's scales: one per head row, or with MX the scales of the two
    // blocks this lane half supplies (blocks 2g + ks at k-step ks)
    int SA[TQ][NMT][MX ? 2 : 1];
    int64_t vis[TQ];
#pragma unroll
    for (int t = 0; t < TQ; ++t) {
        const int row = r0 + (t < nq ? t : 0);
        vis[t] = visible_count(n, q_pos[row], ratio);
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt) {
            // the A row li of slot (t, mt): head 32 mt + li of row t, or with four
            // rows M-tile m = NMT (t % 2) + mt of the row pair t / 2, whose row li
            // holds head 16 m + 4 (li / 8) + li % 4 of row 2 (t / 2) + (li / 4) % 2:
            // the 32x32 product then leaves each lane half the 16 heads of one row
            // of the pair in the order the head sum takes them
            int arow = row, ahead = 32 * mt + li;
            if constexpr (TQ == 4) {
                const int qq = 2 * (t >> 1) + ((li >> 2) & 1);
                arow = r0 + (qq < nq ? qq : 0);
                ahead = 16 * (NMT * (t & 1) + mt) + 4 * (li >> 3) + (li & 3);
            }
            const uint8_t* qr = q + ((int64_t)arow * H + ahead) * 64 + 32 * g;
            A[t][mt][0] = widen(ld16(qr));
            A[t][mt][1] = widen(ld16(qr + 16));
            if constexpr (MX) {
                const uint32_t qs = *reinterpret_cast<const uint32_t*>(q_sc + ((int64_t)arow * H + ahead) * 4);
                SA[t][mt][0] = scale_byte(qs, 2 * g);
                SA[t][mt][1] = scale_byte(qs, 2 * g + 1);
            } else {
                SA[t][mt][0] = q_sc[(int64_t)arow * H + ahead];
            }
        }
    }

    // Two-deep software pipeline over this wave's tiles p_w, p_w + 256, ...:
    // buffers X and Y hold the indexer K of two tiles; a buffer is refilled
    // with the tile after next right after the MFMAs have read it, so two
    // tiles are in flight while the head-sum epilogue of a tile runs.  The
    // refill has no branch: past this wave's last tile it re-reads that tile
    // (a cache hit), and rows past the end of the sequence are clamped to its
    // last row, so no wait on a load is forced before its data is used.
    struct Buf {
        v4i k[2][2];
        uint32_t sc[MX ? 2 : 1];  // with MX: the four block scales of column 32nt + li
    };
    const int n_tiles = p_w < c1 ? (int)((c1 - p_w + 255) / 256) : 0;
    const int64_t p_last = p_w + 256 * (int64_t)(n_tiles - 1);
    auto fetch = [&](Buf& bf, int64_t p0) {
        const uint8_t* kt = k + (e0 + p0) * 64;  // uniform
        const uint32_t last = (uint32_t)(n - 1 - p0 < 63 ? n - 1 - p0 : 63);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const uint32_t r = min((uint32_t)(32 * nt + li), last);
            bf.k[nt][0] = ld16(kt + r * 64 + 32 * g);
            bf.k[nt][1] = ld16(kt + r * 64 + 32 * g + 16);
            if constexpr (MX) bf.sc[nt] = *reinterpret_cast<const uint32_t*>(k_sc + (e0 + p0 + r) * 4);
        }
    };
    // score the tile at p0 from bf, refilling bf with the tile at p_next once
    // the last query's MFMAs have consumed it
    auto tile = [&](Buf& bf, int64_t p0, int64_t p_next) {
        if constexpr (TQ == 4) {
            // row pairs: lane half g of a pair's 32x32 products holds 16 heads of
            // row 2 pr + g (A row mapping above) for positions p0 + li (nt 0) and
            // p0 + 32 + li (nt 1), so the head sums need no exchange between the
            // lane halves; the weights of the lane's row come from LDS
#pragma unroll
            for (int pr = 0; pr < 2; ++pr) {
                if (2 * pr >= nq) break;
                const int qq = 2 * pr + g;
                float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
                for (int m = 0; m < 2 * NMT; ++m) {
                    const int t = 2 * pr + m / NMT, mt = m % NMT;
                    v16f acc[2];
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) {
                        acc[nt] = v16f{};
#pragma unroll
                        for (int ks = 0; ks < 2; ++ks) {
                            if constexpr (MX)
                                acc[nt] = mfma_fp4_mx(A[t][mt][ks], widen(bf.k[nt][ks]), acc[nt], SA[t][mt][ks],
                                                      scale_byte(bf.sc[nt], 2 * g + ks));
                            else
                                acc[nt] = mfma_scaled(A[t][mt][ks], widen(bf.k[nt][ks]), acc[nt], SA[t][mt][0], 4);
                        }
                    }
                    if (m == 2 * NMT - 1 && (2 * pr + 2 >= nq || pr == 1)) fetch(bf, p_next);
                    // heads 16 m .. 16 m + 15 of row qq, in order
                    const v4f* wq = reinterpret_cast<const v4f*>(wl + qq * H + 16 * m);
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) {
                        const v4f wv = wq[q4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            s0 = __builtin_fmaf(wv[i], relu(acc[0][4 * q4 + i]), s0);
                            s1 = __builtin_fmaf(wv[i], relu(acc[1][4 * q4 + i]), s1);
                        }
                    }
                    // as below: the partial sums stay where they are computed
                    asm volatile("" : "+v"(s0), "+v"(s1));
                    __builtin_amdgcn_sched_barrier(0);
                }
                if (qq < nq) {
                    const int64_t vq = vis_pr[pr];
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2) {
                        const int64_t j = p0 + 32 * h2 + li;
                        if (j < n) {
                            const bool visible = j < vq;
                            float sc = -INFINITY;
                            if (visible) {
                                if constexpr (MX) sc = h2 ? s1 : s0;
                                else sc = ldexpf(h2 ? s1 : s0, (int)ekl[p0 - c0 + 32 * h2 + li] - 127);
                            }
                            if constexpr (LOCAL)
                                sl[qq][p0 - c0 + 32 * h2 + li] = sc;
                            else
                                scores[(int64_t)(r0 + qq) * stride + j] = sc;
                            if (HIST && visible) hist16_add(hl + qq * (kHistBins / 2), score_bin(sc));
                        }
                    }
                }
            }
            return;
        }
        const int64_t jl = p0 + lane;
#pragma unroll
        for (int t = 0; t < TQ; ++t) {
            if (t >= nq) break;
            // one group of 32 heads at a time: its MFMAs, then its part of the
            // head sum (32 accumulator registers live instead of 32 NMT)
            float s = 0.0f;
#pragma unroll
            for (int mt = 0; mt < NMT; ++mt) {
                v16f acc[2];
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    acc[nt] = v16f{};
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks) {
                        if constexpr (MX)
                            acc[nt] = mfma_fp4_mx(A[t][mt][ks], widen(bf.k[nt][ks]), acc[nt], SA[t][mt][ks],
                                                  scale_byte(bf.sc[nt], 2 * g + ks));
                        else
                            acc[nt] = mfma_scaled(A[t][mt][ks], widen(bf.k[nt][ks]), acc[nt], SA[t][mt][0], 4);
                    }
                }
                if (mt == NMT - 1 && (t == nq - 1 || t == TQ - 1)) fetch(bf, p_next);
                s = head_sum_32(acc, w + (int64_t)(r0 + t) * H + 32 * mt, s);
                // the partial sum is complete here (not sunk into the guarded
                // store below), and the next group's MFMAs stay after it, so
                // that only one group's accumulators are live at a time
                asm volatile("" : "+v"(s));
                __builtin_amdgcn_sched_barrier(0);
            }
            if (jl < n) {
                const bool visible = jl < vis[t];
                float sc = -INFINITY;
                if (visible) {
                    if constexpr (MX) sc = s;
                    else sc = ldexpf(s, (int)ekl[p0 - c0 + lane] - 127);
                }
                if constexpr (LOCAL)
                    sl[t][p0 - c0 + lane] = sc;
                else
                    scores[(int64_t)(r0 + t) * stride + jl] = sc;
                if (HIST && visible) hist16_add(hl + t * (kHistBins / 2), score_bin(sc));
            }
        }
    };
    // X's loads are issued before Y's, here as in the loop, so that the wait
    // at the top of the loop can leave Y's loads in flight (vmcnt counts in
    // issue order); a wave without tiles reads the chunk's first tile, so that
    // every wave reaches the staging below with the same loads in flight
    Buf X, Y;
    const int64_t p_first = n_tiles > 0 ? p_w : c0;
    fetch(X, p_first);
    __builtin_amdgcn_sched_barrier(0);
    fetch(Y, n_tiles > 1 ? p_w + 256 : p_first);
    __builtin_amdgcn_sched_barrier(0);
    // keep the loads above this point (they would otherwise sink to their first
    // use, behind the staging's wait)
    asm volatile("" ::: "memory");
    if constexpr (!MX) {
#pragma unroll
        for (int j = 0; j < chunk / 256; ++j) ekl[64 * wave + 256 * j + lane] = sb[j];
    }
    if constexpr (TQ == 4) {  // the weights are read by every wave
        if (threadIdx.x < 4 * H) wl[threadIdx.x] = w_own;
        lds_barrier();
    }
    // pairs of tiles, then an odd last one: the loop body has no exit of its
    // own, so every path into the loop header has the same loads in flight
    int i = 0;
    for (; i + 1 < n_tiles; i += 2) {
        const int64_t p0 = p_w + 256 * (int64_t)i;
        tile(X, p0, p0 + 512 <= p_last ? p0 + 512 : p_last);
        tile(Y, p0 + 256, p0 + 768 <= p_last ? p0 + 768 : p_last);
    }
    if (i < n_tiles) tile(X, p_last, p_last);
    if (!HIST) return;
    __syncthreads();
    if constexpr (LOCAL) {
        const int tid = threadIdx.x;
        for (int t = 0; t < TQ && t < nq; ++t) {
            const int row = r0 + t;
            const int64_t nv64 = vis[t] - c0;
            const int nv = nv64 <= 0 ? 0 : (nv64 < c1 - c0 ? (int)nv64 : (int)(c1 - c0));
            const uint32_t kk = (uint32_t)(nv < lo.K ? nv : lo.K);
            // with the chunks' bounds: the row's F chunks whose positions are
            // all visible each hold m = ceil(K / F) positions at or above the
            // bin of their m-th largest score, so the smallest of these F bins
            // is at or below the bin of the row's K-th largest score, and the
            // Top-K pass only looks at list entries from there up
            uint32_t m = 0;
            if (lo.lbins && nv == chunk) {
                const int64_t n_full = vis[t] / chunk;
                m = (uint32_t)(((int64_t)lo.K + n_full - 1) / n_full);
            }
            uint32_t bm;
            const uint32_t bstar = threshold_bin2(PackedBins{hl + t * (kHistBins / 2)}, kk, m, wtot, found, &bm);
            if (m && tid == 0) lo.lbins[(int64_t)row * lo.max_chunks + blockIdx.x] = bm;
            // the chunk's candidates in position order: thread tid owns positions
            // [PER tid, PER tid + PER) of the chunk; one block-wide scan of the
            // per-thread counts places every thread's run in the list, which
            // each thread then writes from its registers
            constexpr int PER = chunk / 256;
            float v[PER];
#pragma unroll
            for (int j = 0; j < PER; j += 4) {
                const v4f x = *reinterpret_cast<const v4f*>(&sl[t][PER * tid + j]);
                v[j] = x[0];
                v[j + 1] = x[1];
                v[j + 2] = x[2];
                v[j + 3] = x[3];
            }
            uint32_t take = 0;
#pragma unroll
            for (int j = 0; j < PER; ++j)
                take |= (uint32_t)(kk > 0 && PER * tid + j < nv && score_bin(v[j]) >= bstar) << j;
            const uint32_t mine = (uint32_t)__popc(take);
            uint32_t off = block_scan_256(mine, wtot) - mine;
            const uint32_t base = wtot[0] + wtot[1] + wtot[2] + wtot[3];
            uint64_t* lr = lo.lists + ((int64_t)row * lo.max_chunks + blockIdx.x) * chunk;
#pragma unroll
            for (int j = 0; j < PER; ++j)
                if ((take >> j) & 1u) lr[off++] = composite(score_key(v[j]), (uint32_t)(c0 + PER * tid + j));
            if (tid == 0) lo.counts[(int64_t)row * lo.max_chunks + blockIdx.x] = base;
            if (lo.bscores) {  // block maxima over the visible positions of the chunk's blocks
                const int64_t nb = (vis[t] + lo.block - 1) / lo.block;
                for (int lb = tid; lb < chunk / lo.block; lb += 256) {
                    const int64_t blk = c0 / lo.block + lb;
                    if (blk >= nb) break;
                    float mx = -INFINITY;
                    for (int j = lb * lo.block; j < (lb + 1) * lo.block && j < nv; ++j) mx = fmaxf(mx, sl[t][j]);
                    lo.bscores[(int64_t)row * lo.bstride + blk] = mx;
                }
            }
            // Only the bins from the chunk's threshold up reach the row's
            // histogram.  The row's threshold bin B is at or above the threshold
            // of every chunk with at least K visible positions (such a chunk
            // alone has K positions at or above its threshold), and a chunk with
            // fewer flushes all its bins, so the row's counts at and above B are
            // complete, which is all the threshold search reads.
            if (hist)  // the fused Top-K builds the row histogram from the lists instead
                hist16_flush(hl + t * (kHistBins / 2), hist + (int64_t)row * kHistBins, kk ? bstar : (uint32_t)kHistBins);
            __syncthreads();  // threshold_bin's LDS scratch is reused by the next row
        }
    } else {
        for (int t = 0; t < TQ && t < nq; ++t)
            hist16_flush(hl + t * (kHistBins / 2), hist + (int64_t)(r0 + t) * kHistBins);
    }
}

// ---------------------------------------------------------------------------
// Candidate (Reindex) scoring: slot s of row r scores entry cand[r][s].
// Grid (slot chunks of 1024, total_q).  Same operand mapping as the decode scan.
// ---------------------------------------------------------------------------
template <int H, bool HIST, bool MX>
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
    int SA[NMT][MX ? 2 : 1];
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
        const uint8_t* qr = q + ((int64_t)row * H + 32 * mt + li) * 64 + 32 * g;
        A[mt][0] = widen(ld16(qr));
        A[mt][1] = widen(ld16(qr + 16));
        if constexpr (MX) {
            const uint32_t qs = *reinterpret_cast<const uint32_t*>(q_sc + ((int64_t)row * H + 32 * mt + li) * 4);
            SA[mt][0] = scale_byte(qs, 2 * g);
            SA[mt][1] = scale_byte(qs, 2 * g + 1);
        } else {
            SA[mt][0] = q_sc[(int64_t)row * H + 32 * mt + li];
        }
    }
    if (HIST) __syncthreads();
    for (int p0 = s0 + 64 * wave; p0 < s1; p0 += 256) {
        v8i B[2][2];
        uint32_t bs[2];  // with MX: the four block scales of column 32nt + li
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            // the list reads are unconditional (clamped to the chunk) so that
            // they are issued together instead of one branch at a time
            const int s = p0 + 32 * nt + li;
            const int32_t cj = crow[s < s1 ? s : s1 - 1];
            int64_t j = s < s1 ? (int64_t)cj : -1;
            j = (j >= 0 && j < vis) ? j : 0;
            const uint8_t* kr = k + (e0 + j) * 64 + 32 * g;
            B[nt][0] = widen(ld16(kr));
            B[nt][1] = widen(ld16(kr + 16));
            if constexpr (MX) bs[nt] = *reinterpret_cast<const uint32_t*>(k_sc + (e0 + j) * 4);
        }
        const int sl = p0 + lane;
        const int32_t cl = crow[sl < s1 ? sl : s1 - 1];
        const int64_t jl = sl < s1 ? (int64_t)cl : -1;
        const bool ok = jl >= 0 && jl < vis;
        int ek = 127;
        if constexpr (!MX) {
            const int e = (int)k_sc[e0 + (ok ? jl : 0)];  // vis > 0: entry 0 exists
            ek = ok ? e : 127;
        }
        v16f acc[NMT][2];
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                acc[mt][nt] = v16f{};
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    if constexpr (MX)
                        acc[mt][nt] = mfma_fp4_mx(A[mt][ks], B[nt][ks], acc[mt][nt], SA[mt][ks], scale_byte(bs[nt], 2 * g + ks));
                    else
                        acc[mt][nt] = mfma_scaled(A[mt][ks], B[nt][ks], acc[mt][nt], SA[mt][0], 4);
                }
            }
        const float sc = head_sum<NMT>(acc, w + (int64_t)row * H);
        if (sl < s1) {
            const float v = ok ? (MX ? sc : ldexpf(sc, ek - 127)) : -INFINITY;
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
template <int H, int QFMT, bool MX>
__global__ __launch_bounds__(256) void k_score_prefill(const uint8_t* __restrict__ q,
                                                       const uint8_t* __restrict__ q_sc,
                                                       const float* __restrict__ w, const uint8_t* __restrict__ k,
                                                       const uint8_t* __restrict__ k_sc,
                                                       const int64_t* __restrict__ entry_off,
                                                       const int32_t* __restrict__ q_off,
                                                       const int32_t* __restrict__ q_pos, int ratio,
                                                       float* __restrict__ scores, int64_t stride,
                                                       uint32_t* __restrict__ tmax, int64_t tstride,
                                                       float* __restrict__ bmax, int64_t bstride) {
    constexpr int NMT = H / 32;
    constexpr int PT = 1024;
    constexpr int QG = 8;
    constexpr int QROW = QFMT == 0 ? 128 : 64;  // bytes per head row
    __shared__ __attribute__((aligned(16))) uint8_t ks_lds[PT * 64];
    __shared__ uint8_t ksc_lds[MX ? 1 : PT];
    __shared__ uint32_t ksc4_lds[MX ? PT : 1];  // with MX: the four block scales of each row
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
        if constexpr (MX)
            ksc4_lds[i] = j < n ? *reinterpret_cast<const uint32_t*>(k_sc + (e0 + j) * 4) : 0x7F7F7F7Fu;
        else
            ksc_lds[i] = j < n ? k_sc[e0 + j] : 127;
    }

    // two query rows per wave, in registers
    v8i A[2][NMT][2];
    // the query's scales: one per head row, or with MX the scales of the two
    // blocks this lane half supplies (block 2ks + g at k-step ks)
    int SA[2][NMT][MX ? 2 : 1];
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
            if constexpr (MX) {
                const uint32_t qs = *reinterpret_cast<const uint32_t*>(q_sc + ((int64_t)row * H + 32 * mt + li) * 4);
                SA[u][mt][0] = scale_byte(qs, g);
                SA[u][mt][1] = scale_byte(qs, 2 + g);
            } else {
                SA[u][mt][0] = q_sc[(int64_t)row * H + 32 * mt + li];
            }
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
        const int ek = MX ? 127 : ksc_lds[64 * tile + lane];
        uint32_t bs[2];
        if constexpr (MX) {
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) bs[nt] = ksc4_lds[64 * tile + 32 * nt + li];
        }
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
                    for (int ks = 0; ks < 2; ++ks) {
                        if constexpr (MX)
                            acc[mt][nt] = mfma_fp4_mx(A[u][mt][ks], B[nt][ks], acc[mt][nt], SA[u][mt][ks],
                                                      scale_byte(bs[nt], 2 * ks + g));
                        else
                            acc[mt][nt] = mfma_scaled(A[u][mt][ks], B[nt][ks], acc[mt][nt], SA[u][mt][0], QFMT == 0 ? 0 : 4);
                    }
                }
            const float s = head_sum<NMT>(acc, w + (int64_t)rows[u] * H);
            const float sv = jl < vis[u] ? (MX ? s : ldexpf(s, ek - 127)) : -INFINITY;
            if (jl < n) scores[(int64_t)rows[u] * stride + jl] = sv;
            if (tmax || bmax) {  // the blocks' and the tile's largest stored scores (lanes past n take no part)
                const float bv = max8(jl < n ? sv : -INFINITY);
                if (bmax && (lane & (kPoolBlock - 1)) == 0) bmax[(int64_t)rows[u] * bstride + jl / kPoolBlock] = bv;
                if (tmax) {
                    const float mv = max64_8(bv);
                    if (lane == 63) tmax[(int64_t)rows[u] * tstride + p0 / kTile] = score_key(mv);
                }
            }
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
// contracts on the bf16 matrix cores.  Every partial sum of a dot product is
// a multiple of the smallest product's grid and below the sum of magnitudes,
// so the channel order inside the contraction does not change the result.
//
// A wave holds two query rows.  The 32 rows of its A operand interleave them
// so that the result's two lane halves belong to different queries: MFMA row
// m holds query (m/4)%2, head 16 mt + 4 (m/8) + m%4, which lands in lane half
// (m/4)%2, register 4 (m/8) + m%4.  So a lane receives 16 consecutive heads of
// its own query for one position, and runs that query's fmaf chain over the
// heads with no cross-lane exchange; its weights come from LDS (the two lane
// halves read two broadcast addresses).  Lane half g supplies channels
// 64 g + 8 ks .. +8 at k-step ks, i.e. bytes 32 g .. 32 g + 31 of an FP4 key
// row, which are read as two 16-byte pieces; the pieces of row p sit at
// piece index c ^ ((p / 2) % 4) in LDS, so that the 8 lanes of each LDS read
// cycle hit distinct banks.  Grid as in k_score_prefill.
// ---------------------------------------------------------------------------
constexpr int kPrefillChunk = 512;       // positions per LDS buffer
constexpr int kPrefillSegChunks = 32;    // chunks per workgroup (16,384 positions)

template <int H>
__global__ __launch_bounds__(256, 2) void k_score_prefill_fp8(const uint8_t* __restrict__ q,
                                                           const uint8_t* __restrict__ q_sc,
                                                           const float* __restrict__ w,
                                                           const uint8_t* __restrict__ k,
                                                           const uint8_t* __restrict__ k_sc,
                                                           const int64_t* __restrict__ entry_off,
                                                           const int32_t* __restrict__ q_off,
                                                           const int32_t* __restrict__ q_pos, int ratio,
                                                           float* __restrict__ scores, int64_t stride,
                                                           uint32_t* __restrict__ tmax, int64_t tstride) {
    constexpr int NM = H / 16;  // MFMA row groups: 16 heads of each of the wave's two queries
    constexpr int PT = kPrefillChunk;
    constexpr int QG = 8;
    __shared__ __attribute__((aligned(16))) uint8_t ks_lds[2][PT * 64];
    __shared__ uint8_t ksc_lds[2][PT];
    __shared__ __attribute__((aligned(16))) float w_lds[QG * H];
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
    // this workgroup's segment: chunks [c_lo, c_hi) of PT positions; the
    // chunks from c_vis on hold no position any of its rows sees
    const int64_t c_lo = (int64_t)blockIdx.x * kPrefillSegChunks;
    const int64_t n_chunks = (n + PT - 1) / PT;
    const int64_t c_hi = c_lo + kPrefillSegChunks < n_chunks ? c_lo + kPrefillSegChunks : n_chunks;
    const int64_t v_chunks = (vmax + PT - 1) / PT;
    const int64_t c_vis = c_hi < v_chunks ? c_hi : v_chunks;
    for (int64_t j = (c_vis > c_lo ? c_vis : c_lo) * PT + threadIdx.x; j < c_hi * PT && j < n; j += 256)
        for (int i = 0; i < nr; ++i) scores[(int64_t)(r0 + i) * stride + j] = -INFINITY;
    if (c_lo >= c_vis) return;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 5, li = lane & 31;

    // 16-byte piece `idx` of a chunk: row idx/4, piece idx%4, stored at piece
    // index (idx%4) ^ ((row/2)%4) of the row
    auto piece_src = [&](int64_t c, int idx) {
        int64_t j = c * PT + (idx >> 2);
        j = j < n ? j : n - 1;
        return k + (e0 + j) * 64 + (idx & 3) * 16;
    };
    auto piece_dst = [&](int buf, int idx) {
        const int row = idx >> 2;
        return ks_lds[buf] + row * 64 + 16 * ((idx & 3) ^ ((row >> 1) & 3));
    };
    for (int i = threadIdx.x; i < PT * 4; i += 256) *reinterpret_cast<v4i*>(piece_dst(0, i)) = ld16(piece_src(c_lo, i));
    for (int i = threadIdx.x; i < PT; i += 256) {
        const int64_t j = c_lo * PT + i;
        ksc_lds[0][i] = j < n ? k_sc[e0 + j] : 127;
    }
    for (int i = threadIdx.x; i < QG * H; i += 256) {
        const int qi = i / H;
        w_lds[i] = w[(int64_t)(qi < nr ? r0 + qi : r0) * H + i % H];
    }

    // A operand: lane li supplies MFMA row li (query (li/4)%2 of the wave)
    v8bf A[NM][8];
    {
        const int qa = 2 * wave + ((li >> 2) & 1);
        const int64_t row = qa < nr ? r0 + qa : r0;
#pragma unroll
        for (int mt = 0; mt < NM; ++mt) {
            const int head = 16 * mt + 4 * (li >> 3) + (li & 3);
            const uint8_t* qr = q + (row * H + head) * 128 + 64 * g;
            const float sc = __builtin_ldexpf(1.0f, (int)q_sc[row * H + head] - 127);
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                const uint2 c = *reinterpret_cast<const uint2*>(qr + 8 * ks);
                auto lo0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.x, sc, false);
                auto lo1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.x, sc, true);
                auto hi0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.y, sc, false);
                auto hi1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.y, sc, true);
                A[mt][ks] = v8bf{lo0[0], lo0[1], lo1[0], lo1[1], hi0[0], hi0[1], hi1[0], hi1[1]};
            }
        }
    }
    // this lane's output query
    const int qo = 2 * wave + g;
    const bool live = qo < nr;
    const int64_t rowo = live ? r0 + qo : r0;
    const int64_t vis = visible_count(n, q_pos[rowo], ratio);
    const float* wq = w_lds + qo * H;

    for (int64_t c = c_lo; c < c_vis; ++c) {
        // chunk c is in buffer (c - c_lo) % 2, and every wave is done with
        // the other buffer, which receives chunk c + 1 one tile at a time
        __syncthreads();
        const int buf = (int)((c - c_lo) & 1);
        const bool next = c + 1 < c_vis;
        const int64_t p_end = (c + 1) * PT < n ? (c + 1) * PT : n;
        for (int tile = 0; tile < PT / 64; ++tile) {
            v4i pf = v4i{};
            uint8_t pfs = 127;
            const int pidx = 256 * tile + threadIdx.x;
            if (next) {
                pf = ld16(piece_src(c + 1, pidx));
                const int64_t js = (c + 1) * PT + 64 * tile + threadIdx.x;
                if (threadIdx.x < 64 && js < n) pfs = k_sc[e0 + js];
            }
            const int64_t p0 = c * PT + 64 * tile;
            if (p0 < p_end) {
                // 2 NM groups (nt, mt) in turn: the contraction of group i
                // runs beside the head sums of group i - 1, and a scheduling
                // barrier between the steps keeps the compiler from hoisting
                // every group's contraction ahead of the sums (which would
                // hold all 2 NM results)
                float s[2] = {0.0f, 0.0f};
                v8bf B[8];
                v16f accp;
#pragma unroll
                for (int i = 0; i <= 2 * NM; ++i) {
                    const int nt = i / NM, mt = i % NM;
                    v16f acc;
                    if (i < 2 * NM) {
                        if (mt == 0) {
                            const int prow = 64 * tile + 32 * nt + li;
                            const uint8_t* kr = ks_lds[buf] + prow * 64;
                            const int sw = (prow >> 1) & 3;
                            const v4i c0 = *reinterpret_cast<const v4i*>(kr + 16 * ((2 * g) ^ sw));
                            const v4i c1 = *reinterpret_cast<const v4i*>(kr + 16 * ((2 * g + 1) ^ sw));
#pragma unroll
                            for (int ks = 0; ks < 8; ++ks) {
                                const uint32_t cw = (uint32_t)(ks < 4 ? c0[ks] : c1[ks - 4]);
                                auto b0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, 1.0f, 0);
                                auto b1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, 1.0f, 1);
                                auto b2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, 1.0f, 2);
                                auto b3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, 1.0f, 3);
                                B[ks] = v8bf{b0[0], b0[1], b1[0], b1[1], b2[0], b2[1], b3[0], b3[1]};
                            }
                        }
                        acc = v16f{};
#pragma unroll
                        for (int ks = 0; ks < 8; ++ks)
                            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[mt][ks], B[ks], acc, 0, 0, 0);
                    }
                    if (i > 0) {
                        const int pn = (i - 1) / NM, pm = (i - 1) % NM;
                        const v4f* wv = reinterpret_cast<const v4f*>(wq + 16 * pm);
                        float t = s[pn];
#pragma unroll
                        for (int j4 = 0; j4 < 4; ++j4) {
                            const v4f ww = wv[j4];
#pragma unroll
                            for (int e = 0; e < 4; ++e) t = __builtin_fmaf(ww[e], relu(accp[4 * j4 + e]), t);
                        }
                        // keeps the sums here rather than sunk into the guarded store
                        asm volatile("" ::"v"(t));
                        s[pn] = t;
                    }
                    accp = acc;
                    __builtin_amdgcn_sched_barrier(0);
                }
                float mv = -INFINITY;  // the tile's largest stored score for this lane half's query
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    const int64_t j = p0 + 32 * nt + li;
                    const int ek = ksc_lds[buf][64 * tile + 32 * nt + li];
                    const float sv = j < vis ? ldexpf(s[nt], ek - 127) : -INFINITY;
                    if (live && j < p_end) scores[rowo * stride + j] = sv;
                    mv = j < p_end ? fmaxf(mv, sv) : mv;
                }
                if (tmax) {
                    mv = max32_8(max8(mv));
                    if (live && li == 31) tmax[rowo * tstride + p0 / kTile] = score_key(mv);
                }
            }
            if (next) {
                *reinterpret_cast<v4i*>(piece_dst(buf ^ 1, pidx)) = pf;
                if (threadIdx.x < 64) ksc_lds[buf ^ 1][64 * tile + threadIdx.x] = pfs;
            }
        }
    }
}

}  // namespace

hipError_t launch_index_score(const ScoreLaunch& a, hipStream_t s) {
    const csa2_batch* b = a.b;
    const bool mx = a.q_fmt == CSA2_Q_MXFP4;  // FP4 queries and keys with an E8M0 per 32 channels
    if (a.cand) {
        dim3 grid((a.cand_stride + 1023) / 1024, a.g.total_q);
#define CSA2_CAND(HH, HI)                                                                                        \
    do { if (mx) CSA2_CAND_M(HH, HI, true); else CSA2_CAND_M(HH, HI, false); } while (0)
#define CSA2_CAND_M(HH, HI, MM)                                                                                  \
    hipExtLaunchKernelGGL((k_score_cand<HH, HI, MM>), grid, dim3(256), 0, s, a.ev_begin, a.ev_end, 0, a.q, a.q_sc, a.w, a.k, a.k_sc,            \
                       b->d_entry_off, b->d_row_seq, b->d_q_pos, b->ratio, a.cand, a.cand_stride, a.scores,      \
                       a.stride, a.hist)
        if (a.H == 64) {
            if (a.hist) CSA2_CAND(64, true); else CSA2_CAND(64, false);
        } else {
            if (a.hist) CSA2_CAND(32, true); else CSA2_CAND(32, false);
        }
#undef CSA2_CAND
#undef CSA2_CAND_M
        return hipGetLastError();
    }
    if (a.q_fmt != CSA2_Q_FP8 && a.g.max_q_per_seq <= 4) {
        const bool one = a.g.max_q_per_seq <= 1;
        const int out = a.local ? kOutLocal : (a.hist ? kOutHist : kOutScores);
        const int chunk = decode_chunk(one ? 1 : 4, out == kOutLocal);
        const LocalOut lo = a.local ? *a.local : LocalOut{};
        dim3 grid((unsigned)((a.g.max_entries + chunk - 1) / chunk), a.g.n_seq);
#define CSA2_DEC(HH, TT, OO)                                                                                     \
    do { if (mx) CSA2_DEC_M(HH, TT, OO, true); else CSA2_DEC_M(HH, TT, OO, false); } while (0)
#define CSA2_DEC_M(HH, TT, OO, MM)                                                                               \
    hipExtLaunchKernelGGL((k_score_decode<HH, TT, OO, MM>), grid, dim3(256), 0, s, a.ev_begin, a.ev_end, 0, a.q, a.q_sc, a.w, a.k, a.k_sc,      \
                       b->d_entry_off, b->d_q_off, b->d_q_pos, b->ratio, a.scores, a.stride, a.hist, lo)
#define CSA2_DEC_T(HH, OO) \
    do { if (one) CSA2_DEC(HH, 1, OO); else CSA2_DEC(HH, 4, OO); } while (0)
#define CSA2_DEC_O(HH)                                                       \
    do {                                                                     \
        if (out == kOutLocal) CSA2_DEC_T(HH, kOutLocal);                     \
        else if (out == kOutHist) CSA2_DEC_T(HH, kOutHist);                  \
        else CSA2_DEC_T(HH, kOutScores);                                     \
    } while (0)
        if (a.H == 64) CSA2_DEC_O(64); else CSA2_DEC_O(32);
#undef CSA2_DEC_O
#undef CSA2_DEC_T
#undef CSA2_DEC
#undef CSA2_DEC_M
        return hipGetLastError();
    }
    if (a.q_fmt == CSA2_Q_FP8) {
        if (a.bmax) return hipErrorInvalidValue;  // block maxima come from the FP4 scorer only
        // one workgroup per (segment of kPrefillSegChunks chunks, 8 rows);
        // consecutive segments go to consecutive XCDs
        constexpr int64_t seg = (int64_t)kPrefillChunk * kPrefillSegChunks;
        dim3 grid((unsigned)((a.g.max_entries + seg - 1) / seg), (unsigned)((a.g.max_q_per_seq + 7) / 8), a.g.n_seq);
        if (a.H == 64)
            hipExtLaunchKernelGGL((k_score_prefill_fp8<64>), grid, dim3(256), 0, s, a.ev_begin, a.ev_end, 0, a.q, a.q_sc, a.w, a.k, a.k_sc,
                               b->d_entry_off, b->d_q_off, b->d_q_pos, b->ratio, a.scores, a.stride, a.tmax, a.tstride);
        else
            hipExtLaunchKernelGGL((k_score_prefill_fp8<32>), grid, dim3(256), 0, s, a.ev_begin, a.ev_end, 0, a.q, a.q_sc, a.w, a.k, a.k_sc,
                               b->d_entry_off, b->d_q_off, b->d_q_pos, b->ratio, a.scores, a.stride, a.tmax, a.tstride);
        return hipGetLastError();
    }
    dim3 grid((unsigned)((a.g.max_entries + 1023) / 1024), (unsigned)((a.g.max_q_per_seq + 7) / 8), a.g.n_seq);
#define CSA2_PRE(HH, FF)                                                                                          \
    do { if (mx) CSA2_PRE_M(HH, FF, true); else CSA2_PRE_M(HH, FF, false); } while (0)
#define CSA2_PRE_M(HH, FF, MM)                                                                                    \
    hipExtLaunchKernelGGL((k_score_prefill<HH, FF, MM>), grid, dim3(256), 0, s, a.ev_begin, a.ev_end, 0, a.q, a.q_sc, a.w, a.k, a.k_sc,          \
                       b->d_entry_off, b->d_q_off, b->d_q_pos, b->ratio, a.scores, a.stride, a.tmax, a.tstride, a.bmax, \
                       a.bstride)
    if (a.H == 64) CSA2_PRE(64, 4); else CSA2_PRE(32, 4);
#undef CSA2_PRE
#undef CSA2_PRE_M
    return hipGetLastError();
}

}  // namespace csa2
