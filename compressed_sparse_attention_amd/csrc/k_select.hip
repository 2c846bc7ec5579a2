// Exact Top-K selection and the hierarchical block pool.
//
// Top-K (report "DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache
// Compression", section 2.3; K = 512 in section 4.2.1): per query row, the
// first min(K, n) slots under (score descending, position ascending), returned
// in ascending position order.  A score maps to an order-preserving unsigned
// key (csa2_internal.h), and the composite
//     key64 = (key << 32) | (0xFFFFFFFF - slot)
// is unique per slot and orders exactly like (score desc, slot asc), so the
// selection is a plain radix select on key64 with no tie cases.
//
// Pass structure (every pass spans many workgroups per row):
//   hist     histogram of score bits 30..19 (4096 bins; negatives in bin 0) per row
//   thresh   per row, the bin that holds the K-th largest score
//   collect  every slot in a bin at or above it -> per-row candidate list
//   final    per row, radix select on key64 among the candidates in LDS,
//            then a bitonic sort of the K winners by slot
//   fallback rows whose candidate list overflowed (heavy ties) are selected
//            straight from the scores with the same radix select and an
//            in-order compaction
//
// Block pool (section 2.3.2; the reading note "DeepSeek V4.1 Flash: Pushing
// the Limits of KV Cache Compression": block selection uses the same position
// scores and is independent of the Top-K): block score = max over the block's
// visible positions; the Top-max_blocks blocks are chosen with the same
// selection (slots = blocks), then expanded to their visible positions.
#include "csa2_internal.h"

namespace csa2 {
namespace {

constexpr int kHChunk = 8192;  // slots per workgroup in the histogram / collect passes
constexpr int kFinalBitmapSlots = 262144;  // rows up to this many slots write their winners through a bitmap

struct RowSrc {
    const int64_t* entry_off;
    const int32_t* row_seq;
    const int32_t* q_pos;
    int ratio;
    const int32_t* cand_count;  // non-null: n = cand_count[row]
    int block_mode, block;
    int64_t max_n;              // slots per row that exist in memory (clamps cand_count)
};

__device__ __forceinline__ int64_t row_n(const RowSrc& rs, int row) {
    if (rs.cand_count) {
        const int64_t c = rs.cand_count[row];
        return c <= 0 ? 0 : (c < rs.max_n ? c : rs.max_n);
    }
    const int b = rs.row_seq[row];
    const int64_t n = rs.entry_off[b + 1] - rs.entry_off[b];
    const int64_t vis = visible_count(n, rs.q_pos[row], rs.ratio);
    return rs.block_mode ? (vis + rs.block - 1) / rs.block : vis;
}

__global__ void k_fill_u32(uint32_t* __restrict__ p, int64_t n, uint32_t v) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = v;
}

// Chunk bounds (rows with no histogram), from every cs-th chunk: workgroup
// (i, row) counts the bins of the slots of chunk c = cs i, [c kHChunk,
// (c+1) kHChunk), in LDS and, when those slots all exist, records the bin of
// their m-th largest score, m = ceil(K / F), F the row's count of such sampled
// full chunks.  The F chunks then hold F m >= K slots at or above the smallest
// recorded bin, so that bin is at or below the row's threshold bin; no global
// atomics are needed.  Sampling reads 1/cs of the scores for a looser bound:
// about cs K slots pass it instead of about K, which the collect pass and the
// final radix select absorb while cs K stays well inside their capacity.
inline int bound_stride(int K) { return K <= 512 ? 4 : (K <= 1024 ? 2 : 1); }
// A row with a tile bound (tb[row] != 0, k_tile_bound) needs no chunk bound.
__global__ __launch_bounds__(256) void k_chunk_bound(const float* __restrict__ scores, int64_t stride, RowSrc rs,
                                                     int K, int cs, const uint32_t* __restrict__ tb,
                                                     uint32_t* __restrict__ lb) {
    __shared__ uint32_t h[kHistBins];
    __shared__ uint32_t wtot[4], found[2];
    const int row = blockIdx.y;
    if (tb && tb[row]) return;
    const int64_t n = row_n(rs, row);
    const int64_t c = (int64_t)blockIdx.x * cs;
    const int64_t s0 = c * kHChunk;
    if (s0 + kHChunk > n) return;  // a partial chunk (or none): no bound
    const int64_t F = (n / kHChunk + cs - 1) / cs;
    const uint32_t m = (uint32_t)((K + F - 1) / F);
    for (int i = threadIdx.x; i < kHistBins; i += 256) h[i] = 0;
    __syncthreads();
    const float* sr = scores + (int64_t)row * stride + s0;
    for (int base = 0; base < kHChunk; base += 256 * 8) {
        uint32_t key[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) key[u] = score_key(sr[base + threadIdx.x + 256 * u]);
#pragma unroll
        for (int u = 0; u < 8; ++u) atomicAdd(&h[key_bin(key[u])], 1u);
    }
    __syncthreads();
    const uint32_t bm = threshold_bin(PlainBins{h}, m, wtot, found);
    if (threadIdx.x == 0) lb[(int64_t)row * kHistBins + c] = bm;
}

// The tile bound of a row from the prefill scorer's tile maxima (the key of
// the largest score of each kTile-slot tile): a key T at most the kk-th
// largest of the row's tile maxima.  Those kk tiles each hold a slot that
// reaches T, so the row's kk-th largest key is at least T, and only the tiles
// whose maximum reaches T hold candidates.  T is the smallest key of the
// 128-key sub-bin (bits 31..7) holding that kk-th largest maximum: its bin
// first, then bits 18..7 within the bin.  tb[row] = 0 (no tile bound) for a
// row of fewer than kk tiles, or when that maximum lies in bin 0 (where keys
// of both signs mix).
constexpr int kTileBatch = 16;  // tile maxima per thread in flight

__global__ __launch_bounds__(256) void k_tile_bound(const uint32_t* __restrict__ tmax, int64_t tstride, RowSrc rs,
                                                    int K, uint32_t* __restrict__ tb) {
    __shared__ uint32_t h[kHistBins];
    __shared__ uint32_t wtot[4], found[2];
    const int row = blockIdx.x;
    const int64_t n = row_n(rs, row);
    const uint32_t kk = (uint32_t)(n < K ? n : K);
    const int64_t nt = (n + kTile - 1) / kTile;
    if (kk == 0 || nt < (int64_t)kk) {
        if (threadIdx.x == 0) tb[row] = 0u;
        return;
    }
    const uint32_t* tr = tmax + (int64_t)row * tstride;
    // count(f): f(key) for each of the row's nt tile maxima, kTileBatch loads
    // per thread issued together (a slot past nt re-reads the last one and
    // is not counted)
    auto count = [&](auto&& f) {
        for (int64_t t0 = 0; t0 < nt; t0 += 256 * kTileBatch) {
            uint32_t k[kTileBatch];
#pragma unroll
            for (int u = 0; u < kTileBatch; ++u) {
                const int64_t t = t0 + threadIdx.x + 256 * u;
                k[u] = tr[t < nt ? t : nt - 1];
            }
#pragma unroll
            for (int u = 0; u < kTileBatch; ++u)
                if (t0 + threadIdx.x + 256 * u < nt) f(k[u]);
        }
    };
    for (int i = threadIdx.x; i < kHistBins; i += 256) h[i] = 0;
    __syncthreads();
    count([&](uint32_t k) { atomicAdd(&h[key_bin(k)], 1u); });
    __syncthreads();
    const uint32_t B = threshold_bin(PlainBins{h}, kk, wtot, found);
    const uint32_t above = found[1];
    if (B == 0) {  // the same for every thread
        if (threadIdx.x == 0) tb[row] = 0u;
        return;
    }
    for (int i = threadIdx.x; i < kHistBins; i += 256) h[i] = 0;
    __syncthreads();
    const uint32_t top = B + 4096u;  // bits 31..19 of every key in bin B
    count([&](uint32_t k) {
        if ((k >> 19) == top) atomicAdd(&h[(k >> 7) & 0xFFFu], 1u);
    });
    __syncthreads();
    const uint32_t subbin = threshold_bin(PlainBins{h}, kk - above, wtot, found);
    if (threadIdx.x == 0) tb[row] = (top << 19) | (subbin << 7);
}

// Candidates: every slot whose bin is at or above the threshold bin goes to
// the row's candidate list.  A workgroup first gathers its candidates in LDS
// and then reserves room in the row's list with a single atomic (a returning
// atomic per wave on one counter would serialise).  A workgroup with more
// candidates than its LDS list holds marks the row as overflowed, which sends
// the row to the exact fallback of k_final.  Every workgroup derives the
// threshold bin from the finished histogram itself; the first workgroup of
// each row records it for the final pass.
constexpr int kLocalCand = 2048;

// LB: `hist` holds the chunk bounds of k_chunk_bound instead of a histogram,
// and the candidates are the slots at or above the smallest of them; or, for
// a row with a tile bound T (tb[row] != 0), the slots whose key reaches T,
// read only from the tiles whose maximum (tmax) reaches it.
template <bool LB>
__global__ __launch_bounds__(256) void k_collect(const float* __restrict__ scores, int64_t stride, RowSrc rs,
                                                 const uint32_t* __restrict__ hist, int K, int cs,
                                                 const uint32_t* __restrict__ tmax, int64_t tstride,
                                                 const uint32_t* __restrict__ tb, RowSel* __restrict__ sel,
                                                 uint64_t* __restrict__ cand_buf) {
    __shared__ uint32_t part[4];
    __shared__ uint32_t found[2];
    __shared__ uint64_t lc[kLocalCand];
    __shared__ uint32_t lcount, gbase;
    __shared__ uint8_t tl[kHChunk / kTile];
    __shared__ uint32_t ntl;
    const int row = blockIdx.y;
    const int64_t n = row_n(rs, row);
    const int64_t s0 = (int64_t)blockIdx.x * kHChunk;
    if (s0 >= n && blockIdx.x != 0) return;
    const float* sr = scores + (int64_t)row * stride;
    const int64_t s1 = s0 + kHChunk < n ? s0 + kHChunk : n;
    const int lane = threadIdx.x & 63;
    // this workgroup's candidates (lcount of them in lc) to the row's list
    auto append = [&]() {
        __syncthreads();
        const uint32_t cnt = lcount;
        if (cnt == 0) return;
        if (threadIdx.x == 0)
            gbase = atomicAdd(&sel[row].cnt, cnt <= (uint32_t)kLocalCand ? cnt : (uint32_t)kCandCap + 1u);
        __syncthreads();
        if (cnt > (uint32_t)kLocalCand) return;  // row overflowed: k_final selects it from the scores
        uint64_t* cb = cand_buf + (int64_t)row * kCandCap;
        for (uint32_t i = threadIdx.x; i < cnt; i += 256)
            if (gbase + i < (uint32_t)kCandCap) cb[gbase + i] = lc[i];
    };
    // put(take, key, slot) for the slots of one pass, the candidates gathered
    // in LDS by one reservation per wave
    auto put = [&](bool take, uint32_t key, int64_t s) {
        const uint64_t m = __ballot(take);
        if (m) {
            uint32_t p0 = 0;
            if (lane == 0) p0 = atomicAdd(&lcount, (uint32_t)__popcll(m));
            p0 = __shfl(p0, 0);
            if (take) {
                const uint32_t p = p0 + (uint32_t)__popcll(m & ((1ull << lane) - 1));
                if (p < (uint32_t)kLocalCand) lc[p] = composite(key, (uint32_t)s);
            }
        }
    };
    if constexpr (LB) {
        const uint32_t T = tb ? tb[row] : 0u;
        if (T) {
            const uint32_t kk = (uint32_t)(n < K ? n : K);
            if (blockIdx.x == 0 && threadIdx.x == 0) {
                sel[row].n = (uint32_t)n;
                sel[row].kk = kk;
                sel[row].bin = key_bin(T);
                sel[row].above = 0u;
                sel[row].lb = 1u;
            }
            if (s0 >= n) return;
            // the chunk's tiles whose maximum reaches T, listed in LDS
            const int64_t t0 = s0 / kTile, nt = (n + kTile - 1) / kTile;
            if (threadIdx.x == 0) {
                lcount = 0;
                ntl = 0;
            }
            __syncthreads();
            if (threadIdx.x < kHChunk / kTile) {
                const int64_t t = t0 + threadIdx.x;
                const bool reach = t < nt && tmax[(int64_t)row * tstride + (t < nt ? t : nt - 1)] >= T;
                const uint64_t m = __ballot(reach);
                uint32_t p0 = 0;
                if (lane == 0 && m) p0 = atomicAdd(&ntl, (uint32_t)__popcll(m));
                p0 = __shfl(p0, 0);
                if (reach) tl[p0 + (uint32_t)__popcll(m & ((1ull << lane) - 1))] = (uint8_t)threadIdx.x;
            }
            __syncthreads();
            // wave w reads listed tiles w, w + 4, ..., kTileBatch / 2 of them a
            // pass, lane l the tile's slot l (a list index past the end
            // re-reads the last tile and is not kept)
            const uint32_t mt = ntl;
            const int wave = threadIdx.x >> 6;
            constexpr int TP = kTileBatch / 2;
            for (uint32_t i0 = (uint32_t)wave; i0 < mt; i0 += 4u * TP) {
                uint32_t key[TP];
                int64_t sl[TP];
#pragma unroll
                for (int u = 0; u < TP; ++u) {
                    const uint32_t i = i0 + 4u * u;
                    sl[u] = s0 + (int64_t)kTile * tl[i < mt ? i : mt - 1] + lane;
                    key[u] = score_key(sr[sl[u] < s1 ? sl[u] : s1 - 1]);
                }
#pragma unroll
                for (int u = 0; u < TP; ++u) put(i0 + 4u * u < mt && sl[u] < s1 && key[u] >= T, key[u], sl[u]);
            }
            append();
            return;
        }
    }
    // issue this thread's loads before the threshold search, all of them
    // unconditionally (a slot past the chunk re-reads its last slot, and every
    // use below checks s < s1): a load whose value is used under a per-lane
    // condition is moved into a branch by the compiler and waited for alone
    uint32_t key[kHChunk / 256];
    if (s1 > s0) {
#pragma unroll
        for (int u = 0; u < kHChunk / 256; ++u) {
            const int64_t s = s0 + threadIdx.x + 256 * u;
            key[u] = score_key(sr[s < s1 ? s : s1 - 1]);
        }
    } else {
#pragma unroll
        for (int u = 0; u < kHChunk / 256; ++u) key[u] = 0u;
    }
    if (threadIdx.x == 0) lcount = 0;
    const uint32_t kk = (uint32_t)(n < K ? n : K);
    uint32_t bin;
    if constexpr (LB) {
        // the smallest bound of the row's sampled full chunks (0 without one);
        // a row with no slot selects nothing
        const int F = (int)(n / kHChunk);
        uint32_t v = 0xFFFFFFFFu;
        for (int c = cs * threadIdx.x; c < F; c += cs * 256) v = min(v, hist[(int64_t)row * kHistBins + c]);
        for (int o = 32; o > 0; o >>= 1) v = min(v, (uint32_t)__shfl_xor(v, o));
        if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
        __syncthreads();
        v = min(min(part[0], part[1]), min(part[2], part[3]));
        bin = kk == 0 ? (uint32_t)kHistBins : (F > 0 ? v : 0u);
    } else {
        bin = threshold_bin(PlainBins{hist + (int64_t)row * kHistBins}, kk, part, found);
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        sel[row].n = (uint32_t)n;
        sel[row].kk = kk;
        sel[row].bin = bin;
        sel[row].above = LB ? 0u : found[1];
        sel[row].lb = LB ? 1u : 0u;
    }
    if (bin >= (uint32_t)kHistBins || s0 >= n) return;
#pragma unroll
    for (int u = 0; u < kHChunk / 256; ++u) {
        const int64_t s = s0 + threadIdx.x + 256 * u;
        put(s < s1 && key_bin(key[u]) >= bin, key[u], s);
    }
    append();
}

// Per row, the threshold bin of its Top-K in the finished histogram (and the
// count above it), recorded in `sel` for the passes over the scan's lists.
__global__ __launch_bounds__(256) void k_row_threshold(const uint32_t* __restrict__ hist, RowSrc rs, int K,
                                                       RowSel* __restrict__ sel) {
    __shared__ uint32_t wtot[4], found[2];
    const int row = blockIdx.x;
    const int64_t n = row_n(rs, row);
    const uint32_t kk = (uint32_t)(n < K ? n : K);
    const uint32_t bin = threshold_bin(PlainBins{hist + (int64_t)row * kHistBins}, kk, wtot, found);
    if (threadIdx.x == 0) {
        sel[row].n = (uint32_t)n;
        sel[row].kk = kk;
        sel[row].bin = bin;
        sel[row].above = found[1];
        sel[row].cnt = 0;
    }
}

// The same filter over a decode scan's per-chunk lists (LocalOut), with the
// row's threshold bin from k_row_threshold.
// Workgroup (c, row) keeps the entries of chunk c's list at or above that bin,
// compacted in place at the front of the list in position order (the list is
// read whole into registers first), and records their count in place of the
// list's.  No atomics: the final pass finds each chunk's run by a prefix sum.
__global__ __launch_bounds__(256) void k_collect_local(uint64_t* __restrict__ lists, uint32_t* __restrict__ counts,
                                                       int max_chunks, int chunk,
                                                       const RowSel* __restrict__ sel) {
    constexpr int U = 4096 / 256;  // entries per thread; chunk <= 4096
    __shared__ uint32_t wtot[4];
    const int row = blockIdx.y;
    uint32_t* cp = counts + (int64_t)row * max_chunks + blockIdx.x;
    uint64_t* lr = lists + ((int64_t)row * max_chunks + blockIdx.x) * chunk;
    // the count is read together with the row state (it is in bounds for every
    // chunk; a chunk past the row's visible range is not used)
    const uint32_t cnt_raw = *cp;
    const RowSel rsel = sel[row];
    const int64_t c0 = (int64_t)blockIdx.x * chunk;
    if (c0 >= (int64_t)rsel.n || rsel.kk == 0) return;  // uniform
    const uint32_t cnt = cnt_raw;
    const uint32_t per = (uint32_t)chunk / 256;  // thread t owns entries [per t, per t + per)
    const uint32_t i0 = per * threadIdx.x;
    uint64_t key[U];
#pragma unroll
    for (int u = 0; u < U; ++u) key[u] = (uint32_t)u < per && i0 + u < cnt ? lr[i0 + u] : 0ull;
    uint32_t take = 0;
#pragma unroll
    for (int u = 0; u < U; ++u)
        take |= (uint32_t)((uint32_t)u < per && i0 + u < cnt && key64_bin(key[u]) >= rsel.bin) << u;
    const uint32_t mine = (uint32_t)__popc(take);
    uint32_t off = block_scan_256(mine, wtot) - mine;  // the barrier inside follows every load
    const uint32_t total = wtot[0] + wtot[1] + wtot[2] + wtot[3];
#pragma unroll
    for (int u = 0; u < U; ++u)
        if ((take >> u) & 1u) lr[off++] = key[u];
    if (threadIdx.x == 0) *cp = total;
}

// Radix select helpers over key64 with 8-bit digits from the top.  `count`
// elements (from LDS or generated) are examined per level; the result is the
// smallest threshold T such that exactly kk elements have key64 >= T.
struct RadixState {
    uint64_t prefix;  // fixed high bits (already shifted down by `shift`)
    int shift;        // bits below the fixed prefix
    uint32_t need;    // elements still to take among those matching the prefix
    int done;
};

// The select state for a candidate set of every key in threshold bin B and
// the bins above it, `above` of them in the bins above (they all win): in a
// bin B >= 1 the keys share their top 13 bits (B + 4096) and the select takes
// kk - above of them from bit 51 down; bin 0 also holds every negative score,
// so the select runs over all candidates from the top bit.
__device__ __forceinline__ void start_in_bin(RadixState* st, uint32_t B, uint32_t kk, uint32_t above) {
    if (B >= 1) {
        st->prefix = (uint64_t)B + 4096u;
        st->shift = 51;
        st->need = kk - above;
    } else {
        st->prefix = 0;
        st->shift = 64;
        st->need = kk;
    }
}

// key64 x against the select state's fixed bits: whether x's bits above
// `sh` equal the prefix (a shift of 64 leaves no fixed bit: every key
// matches), or reach it
__device__ __forceinline__ bool prefix_eq(uint64_t x, int sh, uint64_t pf) { return sh >= 64 || (x >> sh) == pf; }
__device__ __forceinline__ bool prefix_ge(uint64_t x, int sh, uint64_t pf) { return sh >= 64 || (x >> sh) >= pf; }

// digit width at a level: 8 bits, or what realigns `shift` to a multiple of 8
__device__ __forceinline__ int digit_bits(int shift) { return (shift & 7) ? (shift & 7) : 8; }

// Block-wide (every thread of the workgroup calls it, no divergence around the
// barriers): given a 256-bin histogram of the current digit among elements that
// match the fixed prefix, find the digit d with  above(d) < need <= above(d) +
// hist[d]  (above(d) = elements with a larger digit), which is unique, and
// advance the state.
__device__ void radix_step(const uint32_t* hist256, uint32_t* scan256, RadixState* st, int* found) {
    const int t = threadIdx.x;
    if (t < 64) {
        // lane t owns digits 255-4t .. 252-4t; descending exclusive scan
        const int d0 = 255 - 4 * t;
        const uint32_t a = hist256[d0], b = hist256[d0 - 1], c = hist256[d0 - 2], d = hist256[d0 - 3];
        const uint32_t sum = a + b + c + d;
        uint32_t incl = sum;
        for (int off = 1; off < 64; off <<= 1) {
            const uint32_t v = __shfl_up(incl, off);
            if (t >= off) incl += v;
        }
        const uint32_t excl = incl - sum;
        scan256[d0] = excl;
        scan256[d0 - 1] = excl + a;
        scan256[d0 - 2] = excl + a + b;
        scan256[d0 - 3] = excl + a + b + c;
    }
    __syncthreads();
    if (t < 256) {
        const uint32_t above = scan256[t], here = hist256[t];
        if (above < st->need && st->need <= above + here) *found = t;
    }
    __syncthreads();
    if (t == 0) {
        const int d = *found;
        const int w = digit_bits(st->shift);
        const uint32_t above = scan256[d], here = hist256[d];
        st->need -= above;
        st->prefix = (st->prefix << w) | (uint64_t)d;
        st->shift -= w;
        if (here == st->need || st->shift == 0) st->done = 1;
    }
    __syncthreads();
}

__device__ __forceinline__ int32_t map_slot(const int32_t* cand, int cand_stride, int row, uint32_t slot) {
    return cand ? cand[(int64_t)row * cand_stride + slot] : (int32_t)slot;
}

// Inclusive scan of one value per thread over a 1024-thread workgroup; `total`
// receives the workgroup's sum.  Every thread calls it; it ends with a
// barrier, so `wsum` may be reused right after.
__device__ inline uint32_t block_scan_1024(uint32_t v, uint32_t* wsum, uint32_t* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t u = __shfl_up(v, o);
        if (lane >= o) v += u;
    }
    if (lane == 63) wsum[wave] = v;
    __syncthreads();
    uint32_t before = 0, tot = 0;
#pragma unroll
    for (int w2 = 0; w2 < 16; ++w2) {
        const uint32_t x = wsum[w2];
        before += w2 < wave ? x : 0u;
        tot += x;
    }
    *total = tot;
    __syncthreads();
    return before + v;
}

// One workgroup per row: exact selection of the kk winners by key64 and their
// output in ascending position order.  Rows whose candidate list fitted are
// selected from the list in LDS; rows whose list overflowed (heavy ties) are
// selected from all their elements (the same radix select reading them at
// every level, then an in-order compaction).
__global__ __launch_bounds__(1024) void k_final(const float* __restrict__ scores, int64_t stride,
                                                const RowSel* __restrict__ sel, const uint64_t* __restrict__ cand_buf,
                                                const int32_t* __restrict__ cand, int cand_stride, int K,
                                                int32_t* __restrict__ idx) {
    __shared__ uint64_t c[kCandCap];
    __shared__ uint32_t winners[kMaxK];
    __shared__ uint32_t part_rank[512];
    __shared__ uint32_t bmap[kFinalBitmapSlots / 32];  // winners by slot
    __shared__ uint32_t hist256[256], scan256[256];
    __shared__ RadixState st;
    __shared__ uint32_t nwin, base;
    __shared__ int found;
    __shared__ uint32_t wsum[16];
    const int row = blockIdx.x;
    const uint32_t cnt = sel[row].cnt, kk = sel[row].kk;
    const int64_t n = sel[row].n;
    const bool from_list = cnt <= (uint32_t)kCandCap;
    const float* sr = scores + (int64_t)row * stride;
    int32_t* out = idx + (int64_t)row * K;
    for (int i = threadIdx.x + (int)kk; i < K; i += 1024) out[i] = -1;
    if (kk == 0) return;
    if (from_list)
        for (uint32_t i = threadIdx.x; i < cnt; i += 1024) c[i] = cand_buf[(int64_t)row * kCandCap + i];
    if (threadIdx.x == 0) {
        st.prefix = 0;
        st.shift = 64;
        st.need = kk;
        st.done = from_list && cnt == kk;  // every candidate wins
        nwin = 0;
        base = 0;
        if (from_list && !st.done && !sel[row].lb) start_in_bin(&st, sel[row].bin, kk, sel[row].above);
    }
    __syncthreads();
    const int64_t m_elems = from_list ? (int64_t)cnt : n;
    while (!st.done) {
        for (int i = threadIdx.x; i < 256; i += 1024) hist256[i] = 0;
        __syncthreads();
        const int sh = st.shift;
        const int w = digit_bits(sh);
        const uint64_t pf = st.prefix;
        for (int64_t i = threadIdx.x; i < m_elems; i += 1024) {
            const uint64_t x = from_list ? c[i] : composite(score_key(sr[i]), (uint32_t)i);
            const bool m = prefix_eq(x, sh, pf);
            if (m) atomicAdd(&hist256[(uint32_t)(x >> (sh - w)) & ((1u << w) - 1u)], 1u);
        }
        __syncthreads();
        radix_step(hist256, scan256, &st, &found);
    }
    const int sh = st.shift;
    const uint64_t pf = st.prefix;
    if (from_list && n <= kFinalBitmapSlots) {
        // winners (key64 >= prefix << shift) marked by slot, then written in
        // slot order: thread t owns bitmap words [WPT t, WPT (t + 1))
        constexpr int kWpt = kFinalBitmapSlots / 32 / 1024;
        const int nwords = (int)((n + 31) / 32);
        for (int i = threadIdx.x; i < nwords; i += 1024) bmap[i] = 0;
        __syncthreads();
        for (uint32_t i = threadIdx.x; i < cnt; i += 1024) {
            const uint64_t x = c[i];
            if (prefix_ge(x, sh, pf)) {
                const uint32_t slot = 0xFFFFFFFFu - (uint32_t)(x & 0xFFFFFFFFu);
                atomicOr(&bmap[slot >> 5], 1u << (slot & 31));
            }
        }
        __syncthreads();
        const int wpt = (nwords + 1023) / 1024;
        uint32_t wd[kWpt];
        uint32_t wc = 0;
#pragma unroll
        for (int i = 0; i < kWpt; ++i) {
            const int wi = wpt * (int)threadIdx.x + i;
            wd[i] = (i < wpt && wi < nwords) ? bmap[wi] : 0u;
            wc += (uint32_t)__popc(wd[i]);
        }
        uint32_t tot;
        uint32_t r = block_scan_1024(wc, wsum, &tot) - wc;
#pragma unroll
        for (int i = 0; i < kWpt; ++i) {
            uint32_t x = wd[i];
            while (x) {
                const int bit = __ffs(x) - 1;
                if (r < kk) out[r] = map_slot(cand, cand_stride, row, 32u * (uint32_t)(wpt * (int)threadIdx.x + i) + (uint32_t)bit);
                ++r;
                x &= x - 1;
            }
        }
        return;
    }
    if (from_list) {
        // winners: key64 >= prefix << shift; then sort their slots
        for (uint32_t i = threadIdx.x; i < cnt; i += 1024) {
            const uint64_t x = c[i];
            const bool win = prefix_ge(x, sh, pf);
            if (win) {
                const uint32_t p = atomicAdd(&nwin, 1u);
                if (p < (uint32_t)kMaxK) winners[p] = 0xFFFFFFFFu - (uint32_t)(x & 0xFFFFFFFFu);
            }
        }
        __syncthreads();
        // ascending output: a winner's rank is the number of winners with a
        // smaller slot (slots are distinct); the threads of a wave read
        // winners[j] in lock step, so the reads are LDS broadcasts
        const int nw = (int)kk;
        if (nw <= 512) {  // two threads per winner, each counting over half of them
            const int i = threadIdx.x & 511, half = threadIdx.x >> 9;
            const uint32_t my = i < nw ? winners[i] : 0xFFFFFFFFu;
            const int j0 = half ? nw / 2 : 0, j1 = half ? nw : nw / 2;
            uint32_t r = 0;
            for (int j = j0; j < j1; ++j) r += winners[j] < my;
            if (half) part_rank[i] = r;
            __syncthreads();
            if (!half && i < nw) out[r + part_rank[i]] = map_slot(cand, cand_stride, row, my);
            return;
        }
        for (int i0 = 0; i0 < nw; i0 += 1024) {
            const int i = i0 + (int)threadIdx.x;
            const uint32_t my = i < nw ? winners[i] : 0xFFFFFFFFu;
            int rank = 0;
            for (int j = 0; j < nw; ++j) rank += winners[j] < my;
            if (i < nw) out[rank] = map_slot(cand, cand_stride, row, my);
        }
        return;
    }
    // overflowed row: in-order compaction over all slots
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int64_t s0 = 0; s0 < n; s0 += 1024) {
        const int64_t s = s0 + threadIdx.x;
        bool win = false;
        if (s < n) {
            const uint64_t x = composite(score_key(sr[s]), (uint32_t)s);
            win = prefix_ge(x, sh, pf);
        }
        const uint64_t m = __ballot(win);
        if (lane == 0) wsum[wave] = (uint32_t)__popcll(m);
        __syncthreads();
        uint32_t off = base;
        for (int w2 = 0; w2 < wave; ++w2) off += wsum[w2];
        if (win) {
            const uint32_t p = off + (uint32_t)__popcll(m & ((1ull << lane) - 1));
            if (p < kk) out[p] = map_slot(cand, cand_stride, row, (uint32_t)s);
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            uint32_t tot = 0;
            for (int w2 = 0; w2 < 16; ++w2) tot += wsum[w2];
            base += tot;
        }
        __syncthreads();
    }
}

// Final selection from the compacted per-chunk lists (k_collect_local): one
// workgroup per row.  The chunks' runs are concatenated in chunk order into
// LDS, which puts the candidates in position order; the radix select starts
// at bit 51 over the threshold bin's keys (the bins above all win), and the
// winners are written out in that same order by a running compaction, so no
// sort is needed.  A row with more candidates than LDS holds streams them
// from the lists at every step instead.
constexpr int kMaxChunksLds = 4096;  // chunks whose run offsets fit in LDS

__global__ __launch_bounds__(1024) void k_final_local(const uint64_t* __restrict__ lists,
                                                      const uint32_t* __restrict__ counts, int max_chunks,
                                                      int chunk, const RowSel* __restrict__ sel, int K,
                                                      int32_t* __restrict__ idx) {
    __shared__ uint64_t c[kCandCap];
    __shared__ uint32_t roff[kMaxChunksLds + 1];
    __shared__ uint32_t hist256[256], scan256[256];
    __shared__ RadixState st;
    __shared__ int found;
    __shared__ uint32_t wsum[16];
    __shared__ uint32_t base;
    const int row = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint32_t* cr = counts + (int64_t)row * max_chunks;
    // the first 1024 run lengths are read together with the row state
    const uint32_t len0 = tid < max_chunks ? cr[tid] : 0u;
    const RowSel rsel = sel[row];
    const uint32_t kk = rsel.kk;
    int32_t* out = idx + (int64_t)row * K;
    for (int i = tid + (int)kk; i < K; i += 1024) out[i] = -1;
    if (kk == 0) return;
    const int n_ch = (int)(((int64_t)rsel.n + chunk - 1) / chunk);
    const uint64_t* lrow = lists + (int64_t)row * max_chunks * chunk;
    const bool in_lds_offsets = n_ch <= kMaxChunksLds;
    // run offsets: exclusive prefix sum of the runs' lengths
    if (in_lds_offsets) {
        if (tid == 0) base = 0;
        __syncthreads();
        for (int c0 = 0; c0 < n_ch; c0 += 1024) {
            const int ch = c0 + tid;
            const uint32_t v = ch < n_ch ? (c0 == 0 ? len0 : cr[ch]) : 0u;
            uint32_t incl = v;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const uint32_t u = __shfl_up(incl, o);
                if (lane >= o) incl += u;
            }
            if (lane == 63) wsum[wave] = incl;
            __syncthreads();
            uint32_t before = base;
            for (int w2 = 0; w2 < wave; ++w2) before += wsum[w2];
            if (ch < n_ch) roff[ch] = before + incl - v;
            __syncthreads();
            if (tid == 0) {
                uint32_t tot = 0;
                for (int w2 = 0; w2 < 16; ++w2) tot += wsum[w2];
                base += tot;
            }
            __syncthreads();
        }
        if (tid == 0) roff[n_ch] = base;
        __syncthreads();
    }
    const uint32_t total = in_lds_offsets ? roff[n_ch] : 0xFFFFFFFFu;
    const bool from_lds = total <= (uint32_t)kCandCap;
    // element e of the concatenation (e < total): chunk by binary search
    auto elem = [&](uint32_t e) -> uint64_t {
        int lo = 0, hi = n_ch;  // roff[lo] <= e < roff[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (roff[mid] <= e) lo = mid; else hi = mid;
        }
        return lrow[(int64_t)lo * chunk + (e - roff[lo])];
    };
    if (from_lds)
        for (uint32_t e = tid; e < total; e += 1024) c[e] = elem(e);
    if (tid == 0) {
        start_in_bin(&st, rsel.bin, kk, rsel.above);
        st.done = 0;
        base = 0;
    }
    __syncthreads();
    // visit every candidate: from LDS, or streamed from the runs (chunk order)
    auto for_each = [&](auto&& fn) {
        if (from_lds) {
            for (uint32_t e = tid; e < total; e += 1024) fn(c[e]);
        } else {
            for (int ch = 0; ch < n_ch; ++ch) {
                const uint32_t cn = cr[ch];
                for (uint32_t j = tid; j < cn; j += 1024) fn(lrow[(int64_t)ch * chunk + j]);
            }
        }
    };
    while (!st.done) {
        if (tid < 256) hist256[tid] = 0;
        __syncthreads();
        const int sh = st.shift;
        const int w = digit_bits(sh);
        const uint64_t pf = st.prefix;
        for_each([&](uint64_t x) {
            if (prefix_eq(x, sh, pf)) atomicAdd(&hist256[(uint32_t)(x >> (sh - w)) & ((1u << w) - 1u)], 1u);
        });
        __syncthreads();
        radix_step(hist256, scan256, &st, &found);
    }
    const int sh = st.shift;
    const uint64_t pf = st.prefix;
    // winners (key64 >= prefix << shift) in candidate order = position order
    auto emit = [&](uint64_t x, bool valid) {
        const bool win = valid && prefix_ge(x, sh, pf);
        const uint64_t m = __ballot(win);
        if (lane == 0) wsum[wave] = (uint32_t)__popcll(m);
        __syncthreads();
        uint32_t off = base;
        for (int w2 = 0; w2 < wave; ++w2) off += wsum[w2];
        if (win) {
            const uint32_t p = off + (uint32_t)__popcll(m & ((1ull << lane) - 1));
            if (p < kk) out[p] = (int32_t)(0xFFFFFFFFu - (uint32_t)(x & 0xFFFFFFFFu));
        }
        __syncthreads();
        if (tid == 0) {
            uint32_t tot = 0;
            for (int w2 = 0; w2 < 16; ++w2) tot += wsum[w2];
            base += tot;
        }
        __syncthreads();
    };
    if (from_lds) {
        for (uint32_t e0 = 0; e0 < total; e0 += 1024) {
            const uint32_t e = e0 + tid;
            emit(e < total ? c[e] : 0ull, e < total);
        }
    } else {
        for (int ch = 0; ch < n_ch; ++ch) {
            const uint32_t cn = cr[ch];
            for (uint32_t j0 = 0; j0 < cn; j0 += 1024) {
                const uint32_t j = j0 + tid;
                emit(j < cn ? lrow[(int64_t)ch * chunk + j] : 0ull, j < cn);
            }
        }
    }
}


// Block-wide (1024 threads, every thread calls it): the bin (bits 30..19 of
// a score) that holds the kk-th largest of the entries visit() enumerates,
// and the count of entries in the bins above it.  visit(f) calls f(bin) for
// each of this thread's entries.  Two 6-bit digits (bin = 64 d1 + d2), each
// counted into 32 copies of a 64-entry LDS histogram (lane l adds to copy
// l % 32: the entries crowd into a few bins and same-address LDS atomics
// serialise); thr[0..1] must be zero on entry.
template <class Visit>
__device__ void find_bin(Visit&& visit, uint32_t kk, uint32_t* hcopy, uint32_t* dcount, uint32_t* thr, uint32_t& B,
                         uint32_t& above) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint32_t need = kk;
    B = 0;
    above = 0;
#pragma unroll
    for (int level = 0; level < 2; ++level) {
        for (int i = tid; i < 64 * 32; i += 1024) hcopy[i] = 0;
        __syncthreads();
        uint32_t* hc = hcopy + (lane & 31);
        visit([&](uint32_t bin) {
            if (level == 0 || (bin >> 6) == B) atomicAdd(&hc[32 * (level == 0 ? bin >> 6 : bin & 63u)], 1u);
        });
        __syncthreads();
        {  // digit d = tid / 16 sums copies 2 (tid % 16), +1; 16 lanes reduce
            const int d = tid >> 4, part = tid & 15;
            uint32_t v = hcopy[32 * d + 2 * part] + hcopy[32 * d + 2 * part + 1];
#pragma unroll
            for (int o = 8; o > 0; o >>= 1) v += __shfl_xor(v, o, 16);
            if (part == 0) dcount[d] = v;
        }
        __syncthreads();
        if (wave == 0) {  // lane l owns digit 63 - l; inclusive scan from the top
            const uint32_t v = dcount[63 - lane];
            uint32_t incl = v;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const uint32_t u2 = __shfl_up(incl, o);
                if (lane >= o) incl += u2;
            }
            const uint32_t before = incl - v;
            if (before < need && need <= incl) {
                thr[0] = (uint32_t)(63 - lane);
                thr[1] = before;
            }
        }
        __syncthreads();
        B = level == 0 ? thr[0] : (B << 6) | thr[0];
        above += thr[1];
        need -= thr[1];
        __syncthreads();  // thr and hcopy are rewritten by the next level
    }
}

// The whole selection of a row from a decode scan's per-chunk lists, in one
// workgroup of 1024 threads per row and without a histogram from the scan.
// The histogram of the row's threshold search is built from the lists: a
// chunk's list holds exactly its visible positions at or above the chunk's
// threshold bin, and the row's threshold bin B lies at or above the threshold
// of every chunk with K visible positions (a chunk with fewer lists all its
// positions), so the lists hold every position of the row at or above B and
// their histogram has the row's exact counts from B up, which is all the
// search reads.
//
// With the filter's parts (below) the row's entries at or above its bound
// come from them straight into LDS and are selected there; only when a part
// overflowed, or they do not fit, are the lists read, as follows.
//
// The lists are read as their concatenation (chunk order = position order).
// When they hold at most kListWindow entries, thread t keeps entries t,
// t + 1024, ... in registers and they are read once; otherwise every step
// streams them from memory again, chunk by chunk.
//   0. with the chunks' bounds, the entries at or above LB into LDS and the
//      select there, while they fit; else
//   1. B in two 6-bit digits (bin = 64 d1 + d2), each counted into 32 copies
//      of a 64-entry LDS histogram (lane l adds to copy l % 32: the entries
//      crowd into a few bins and same-address LDS atomics serialise);
//   2. the entries at or above B, compacted into LDS in order (or, past
//      kCandCap of them, left in the lists and filtered at every later step);
//   3. radix select of the threshold bin's keys from bit 51 down (the bins
//      above B all win);
//   4. the winners, written in order.
constexpr int kListPer = 22;                    // list entries per thread held in registers
constexpr int kListWindow = 1024 * kListPer;    // 22,528 entries
constexpr int kCandPer = kCandCap / 1024;       // LDS candidates per thread in step 4
constexpr int kSpecParts = 4;                   // filter parts per wave loaded with their counts

// With the chunks' bounds, the entries that survive the bound are gathered by
// many workgroups first (k_lists_filter), so that no single compute unit has
// to pull a whole row's lists: workgroup (g, row) reads the lists of the row's
// chunks [kPartChunks g, kPartChunks (g + 1)), keeps the entries whose bin is
// at or above the row's bound LB (the smallest bound of its full chunks, 0
// without one) and writes them, in any order, to part g of the row's
// candidate buffer (cap entries from g cap), and their count to
// part_cnt[row][g].  A count above cap means the part overflowed (only its
// first cap entries were written): k_topk_lists then selects from the lists.
// Workgroup (0, row) also writes the row's size to part_n[row], so that the
// selection reads it with the counts.
constexpr int kPartChunks = 2;   // list chunks per filter workgroup
constexpr int kPartPer = 8;      // entries per thread per pass past the first
constexpr int kSpecPer = 3;      // entries per thread of each list loaded with the lengths (768 of a list)
constexpr int kMaxParts = 64;    // parts per row (one wave scans their counts)

__global__ __launch_bounds__(256) void k_lists_filter(const uint64_t* __restrict__ lists,
                                                      const uint32_t* __restrict__ counts,
                                                      const uint32_t* __restrict__ lbins, int max_chunks, int chunk,
                                                      RowSrc rs, int cap, uint32_t* __restrict__ part_cnt,
                                                      uint32_t* __restrict__ part_n, uint64_t* __restrict__ part_keys) {
    __shared__ uint32_t wmin[4];
    __shared__ uint32_t nsurv;
    const int row = blockIdx.y, g = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63;
    const int c0 = g * kPartChunks;
    // loaded before the row's size is known, all at once (every address is in
    // the row's lists; what lies past the visible chunks is not used): the
    // lengths of this part's lists, the first 256 kSpecPer slots of each (a
    // list has room for `chunk` >= 256 kSpecPer entries; slots past its
    // length are unused) and the chunks' bounds (max_chunks <= 256)
    const uint64_t* lp = lists + ((int64_t)row * max_chunks + c0) * chunk;
    uint32_t cn[kPartChunks];
    uint64_t xs[kPartChunks][kSpecPer];
#pragma unroll
    for (int i = 0; i < kPartChunks; ++i) {
        const bool in = c0 + i < max_chunks;
        cn[i] = in ? counts[(int64_t)row * max_chunks + c0 + i] : 0u;
#pragma unroll
        for (int u = 0; u < kSpecPer; ++u) xs[i][u] = in ? lp[(int64_t)i * chunk + tid + 256 * u] : 0ull;
    }
    const uint32_t lbv = tid < max_chunks ? lbins[(int64_t)row * max_chunks + tid] : 0xFFFFFFFFu;
    const int64_t n = row_n(rs, row);
    const int n_ch = (int)((n + chunk - 1) / chunk);
    const int n_full = (int)(n / chunk);
    if (g == 0 && tid == 0) part_n[row] = (uint32_t)n;
    uint32_t* cnt_out = part_cnt + (int64_t)row * gridDim.x + g;
    if (c0 >= n_ch) {  // past the row's chunks (or an empty row): an empty part
        if (tid == 0) *cnt_out = 0u;
        return;
    }
#pragma unroll
    for (int i = 0; i < kPartChunks; ++i) cn[i] = c0 + i < n_ch ? cn[i] : 0u;
    uint32_t v = tid < n_full ? lbv : 0xFFFFFFFFu;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = min(v, (uint32_t)__shfl_xor(v, o));
    if (lane == 0) wmin[tid >> 6] = v;
    if (tid == 0) nsurv = 0u;
    __syncthreads();
    const uint32_t LB = n_full > 0 ? min(min(wmin[0], wmin[1]), min(wmin[2], wmin[3])) : 0u;
    uint64_t* dst = part_keys + (int64_t)row * kCandCap + (int64_t)g * cap;
    // the loaded slots: every keep first, then one reservation per wave
    {
        uint32_t keep = 0;
#pragma unroll
        for (int i = 0; i < kPartChunks; ++i)
#pragma unroll
            for (int u = 0; u < kSpecPer; ++u)
                keep |= (uint32_t)((uint32_t)(tid + 256 * u) < cn[i] && key64_bin(xs[i][u]) >= LB)
                        << (i * kSpecPer + u);
        const uint32_t mine = (uint32_t)__popc(keep);
        uint32_t incl = mine;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const uint32_t w = __shfl_up(incl, o);
            if (lane >= o) incl += w;
        }
        uint32_t base = 0;
        if (lane == 63 && incl) base = atomicAdd(&nsurv, incl);
        uint32_t p = __shfl(base, 63) + incl - mine;
#pragma unroll
        for (int i = 0; i < kPartChunks; ++i)
#pragma unroll
            for (int u = 0; u < kSpecPer; ++u)
                if ((keep >> (i * kSpecPer + u)) & 1u) {
                    if (p < (uint32_t)cap) dst[p] = xs[i][u];
                    ++p;
                }
    }
    // the rest of each list, a pass of kPartPer loads per thread at a time (a
    // slot past the list re-reads its last entry; each use checks j < cn)
    auto emit = [&](bool take, uint64_t x) {
        const uint64_t m = __ballot(take);
        if (m) {
            uint32_t p0 = 0;
            if (lane == 0) p0 = atomicAdd(&nsurv, (uint32_t)__popcll(m));
            p0 = __shfl(p0, 0);
            const uint32_t p = p0 + (uint32_t)__popcll(m & ((1ull << lane) - 1));
            if (take && p < (uint32_t)cap) dst[p] = x;
        }
    };
#pragma unroll
    for (int i = 0; i < kPartChunks; ++i) {
        for (uint32_t j0 = 256u * kSpecPer; j0 < cn[i]; j0 += 256u * kPartPer) {
            uint64_t x[kPartPer];
#pragma unroll
            for (int u = 0; u < kPartPer; ++u) {
                const uint32_t j = j0 + (uint32_t)tid + 256u * u;
                x[u] = lp[(int64_t)i * chunk + (j < cn[i] ? j : cn[i] - 1u)];
            }
#pragma unroll
            for (int u = 0; u < kPartPer; ++u)
                emit(j0 + (uint32_t)tid + 256u * u < cn[i] && key64_bin(x[u]) >= LB, x[u]);
        }
    }
    __syncthreads();
    if (tid == 0) *cnt_out = nsurv;
}

__global__ __launch_bounds__(1024) void k_topk_lists(const uint64_t* __restrict__ lists,
                                                     const uint32_t* __restrict__ counts,
                                                     const uint32_t* __restrict__ lbins, int max_chunks, int chunk,
                                                     RowSrc rs, int K, const uint32_t* __restrict__ part_cnt,
                                                     const uint32_t* __restrict__ part_n,
                                                     const uint64_t* __restrict__ part_keys, int parts, int cap,
                                                     int32_t* __restrict__ idx) {
    __shared__ uint64_t c[kCandCap];
    __shared__ uint32_t bm[kFusedTopkEntries / 32];  // winners by position
    __shared__ uint32_t nsurv, lb_sh;
    __shared__ uint32_t hcopy[64 * 32];
    __shared__ uint32_t dcount[64];
    __shared__ uint32_t roff[kListChunks + 1];
    __shared__ uint32_t pcnt[16 * kListPer];
    __shared__ uint32_t hist256[256], scan256[256];
    __shared__ RadixState st;
    __shared__ int found;
    __shared__ uint32_t wsum[16];
    __shared__ uint32_t thr[3];
    __shared__ uint32_t h4k[2 * kHistBins];
    __shared__ uint32_t pover;
    const int row = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // loaded at once: with parts, their counts (parts <= kMaxParts), the
    // row's size and the first slots of each wave's parts; without, the
    // row's size with the lists' lengths and bounds (every chunk of the row
    // is in bounds; those past the visible range are unused)
    uint32_t pc = 0u;
    uint64_t ys[kSpecParts][2];
    uint32_t cnt_raw = 0u, lb_raw = 0xFFFFFFFFu;
    int64_t n;
    if (part_cnt) {
        pc = tid < parts ? part_cnt[(int64_t)row * parts + tid] : 0u;
#pragma unroll
        for (int r = 0; r < kSpecParts; ++r) {
            const int q = wave + 16 * r;  // the same for the whole wave
#pragma unroll
            for (int v = 0; v < 2; ++v)
                ys[r][v] = q < parts ? part_keys[(int64_t)row * kCandCap + (int64_t)q * cap + min(lane + 64 * v, cap - 1)]
                                     : 0ull;
        }
        n = (int64_t)part_n[row];
    } else {
        cnt_raw = tid < max_chunks ? counts[(int64_t)row * max_chunks + tid] : 0u;
        lb_raw = (lbins && tid < max_chunks) ? lbins[(int64_t)row * max_chunks + tid] : 0xFFFFFFFFu;
        n = row_n(rs, row);
    }
    const uint32_t kk = (uint32_t)(n < K ? n : K);
    int32_t* out = idx + (int64_t)row * K;
    for (int i = tid + (int)kk; i < K; i += 1024) out[i] = -1;
    if (kk == 0) return;
    const int n_ch = (int)((n + chunk - 1) / chunk);  // <= max_chunks <= kListChunks (launcher)
    const uint64_t* lrow = lists + (int64_t)row * max_chunks * chunk;
    const int n_full = (int)(n / chunk);  // chunks whose positions are all visible
    if (tid == 0) {
        thr[0] = 0;
        thr[1] = 0;
        nsurv = 0;
        lb_sh = 0xFFFFFFFFu;
    }
    for (int i = tid; i < kFusedTopkEntries / 32; i += 1024) bm[i] = 0;
    for (int i = tid; i < 2 * kHistBins; i += 1024) h4k[i] = 0;
    if (part_cnt && wave == 0) {  // the parts' offsets, and whether one overflowed
        uint32_t incl = pc;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const uint32_t w = __shfl_up(incl, o);
            if (lane >= o) incl += w;
        }
        if (lane < parts) roff[lane] = incl - pc;
        if (lane == 63) roff[parts] = incl;  // lanes at or past `parts` hold 0
        const uint64_t ov = __ballot(lane < parts && pc > (uint32_t)cap);
        if (lane == 0) pover = ov ? 1u : 0u;
    }
    __syncthreads();  // the cleared LDS, the parts' offsets and lb_sh (before any thread lowers it)

    // The K winners among the n_surv keys in c (every key at or above the
    // row's bound, in any order): a radix select on key64 from the top with
    // 12-bit digits, each digit's histogram in 4096 LDS bins (two of them,
    // cleared at the start, one cleared while the other counts), read from
    // the top by a block-wide scan; it stops once every key left with the
    // chosen prefix wins (two digits for distinct scores).  When no key is
    // negative (nonneg) the top bit is fixed and the first digit is the
    // score's bin; `counted`: the caller has counted that first histogram
    // (bins of every key) into h4k and passed a barrier.  The winners are marked in a bitmap by position and
    // written in position order.
    auto mark = [&](uint64_t x) {
        const uint32_t pos = 0xFFFFFFFFu - (uint32_t)(x & 0xFFFFFFFFu);
        atomicOr(&bm[pos >> 5], 1u << (pos & 31));
    };
    auto select_in_lds = [&](uint32_t n_surv, bool nonneg, bool counted) {
        uint64_t pf = nonneg ? 1u : 0u;  // every key's top bit is set: the first digit is its bin
        int sh = nonneg ? 63 : 64;
        uint32_t need = kk;
        for (int pass = 0;; ++pass) {
            uint32_t* h = h4k + (pass & 1) * kHistBins;
            const int w = sh < 12 ? sh : 12;
            if (pass > 0 || !counted) {
                for (uint32_t e = tid; e < n_surv; e += 1024) {
                    const uint64_t x = c[e];
                    if (prefix_eq(x, sh, pf)) atomicAdd(&h[(uint32_t)(x >> (sh - w)) & ((1u << w) - 1u)], 1u);
                }
                __syncthreads();
            }
            {
                // thread t owns digits top .. top - 3 (t = 0 the highest)
                const int top = kHistBins - 1 - 4 * tid;
                uint32_t hb[4], sum = 0;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    hb[i] = h[top - i];
                    sum += hb[i];
                }
                uint32_t tot;
                const uint32_t incl = block_scan_1024(sum, wsum, &tot);
                uint32_t acc = incl - sum;
                if (acc < need && need <= incl) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        if (acc < need && need <= acc + hb[i]) {
                            thr[0] = (uint32_t)(top - i);
                            thr[1] = acc;
                            thr[2] = hb[i];
                        }
                        acc += hb[i];
                    }
                }
            }
            __syncthreads();
            const uint32_t d = thr[0], above = thr[1], here = thr[2];
            for (int i = tid; i < kHistBins; i += 1024) h[i] = 0;  // counted into again two passes on
            need -= above;
            pf = (pf << w) | d;
            sh -= w;
            if (here == need || sh == 0) break;
        }
        for (uint32_t e = tid; e < n_surv; e += 1024) {
            const uint64_t x = c[e];
            if (prefix_ge(x, sh, pf)) mark(x);
        }
        __syncthreads();
        // positions in order: thread t owns bitmap words [WPT t, WPT (t + 1))
        constexpr int kMaxWpt = kFusedTopkEntries / 32 / 1024;
        const int nwords = (int)((n + 31) / 32);
        const int WPT = (nwords + 1023) / 1024;
        uint32_t wd[kMaxWpt];
        uint32_t cnt = 0;
#pragma unroll
        for (int i = 0; i < kMaxWpt; ++i) {
            const int wi = WPT * tid + i;
            wd[i] = (i < WPT && wi < nwords) ? bm[wi] : 0u;
            cnt += (uint32_t)__popc(wd[i]);
        }
        uint32_t tot;
        uint32_t r = block_scan_1024(cnt, wsum, &tot) - cnt;
#pragma unroll
        for (int i = 0; i < kMaxWpt; ++i) {
            uint32_t x = wd[i];
            while (x) {
                const int bit = __ffs(x) - 1;
                if (r < kk) out[r] = 32 * (WPT * tid + i) + bit;
                ++r;
                x &= x - 1;
            }
        }
    };

    // the filter's parts: their entries to LDS when no part overflowed and
    // they fit, then the select; else the lists are read below.  The first
    // kSpecParts parts of each wave (w, w + 16, ...) had their first 128
    // slots loaded with the counts (slots past a part's count are unused)
    if (part_cnt) {
        const uint32_t tot = roff[parts];
        if (!pover && tot <= (uint32_t)kCandCap) {
            // wave w copies parts w, w + 16, ...: the loaded slots first, then
            // the rest four loads per lane at a time (a slot past the part
            // re-reads its last entry)
            bool neg = false;  // a key whose top bit is clear (a negative score)
            auto copy_rest = [&](int q, uint32_t from) {
                const uint32_t b0 = roff[q], cq = roff[q + 1] - b0;
                const uint64_t* src = part_keys + (int64_t)row * kCandCap + (int64_t)q * cap;
                for (uint32_t j0 = from; j0 < cq; j0 += 256) {
                    uint64_t x[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const uint32_t j = j0 + (uint32_t)lane + 64u * u;
                        x[u] = src[j < cq ? j : cq - 1u];
                    }
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const uint32_t j = j0 + (uint32_t)lane + 64u * u;
                        if (j < cq) {
                            c[b0 + j] = x[u];
                            neg |= (x[u] >> 63) == 0;
                            atomicAdd(&h4k[(uint32_t)(x[u] >> 51) & 0xFFFu], 1u);
                        }
                    }
                }
            };
#pragma unroll
            for (int r = 0; r < kSpecParts; ++r) {
                const int q = wave + 16 * r;
                if (q < parts) {
                    const uint32_t b0 = roff[q], cq = roff[q + 1] - b0;
                    const uint32_t have = min(128u, (uint32_t)cap);
#pragma unroll
                    for (int v = 0; v < 2; ++v) {
                        const uint32_t j = (uint32_t)(lane + 64 * v);
                        if (j < cq && j < have) {
                            c[b0 + j] = ys[r][v];
                            neg |= (ys[r][v] >> 63) == 0;
                            atomicAdd(&h4k[(uint32_t)(ys[r][v] >> 51) & 0xFFFu], 1u);
                        }
                    }
                    copy_rest(q, have);
                }
            }
            for (int q = wave + 16 * kSpecParts; q < parts; q += 16) copy_rest(q, 0u);
            // the first histogram (bits 62..51: the bin when no key is
            // negative) was counted with the copy; with a negative key the
            // select starts from the top bit and counts it again
            const bool any_neg = __syncthreads_or(neg) != 0;
            if (any_neg) {
                for (int i = tid; i < kHistBins; i += 1024) h4k[i] = 0;
                __syncthreads();
            }
            select_in_lds(tot, !any_neg, !any_neg);
            return;
        }
        // roff is rewritten below, after the barrier in the scan
        cnt_raw = tid < max_chunks ? counts[(int64_t)row * max_chunks + tid] : 0u;
        lb_raw = (lbins && tid < max_chunks) ? lbins[(int64_t)row * max_chunks + tid] : 0xFFFFFFFFu;
    }
    // run offsets: exclusive prefix sum of the lists' lengths; the lower
    // bound LB of the row's threshold bin: the smallest of the full chunks'
    // bounds (0 when there is no full chunk)
    {
        const uint32_t v = tid < n_ch ? cnt_raw : 0u;
        if (tid < n_full) atomicMin(&lb_sh, lb_raw);
        uint32_t tot;
        const uint32_t incl = block_scan_1024(v, wsum, &tot);
        if (tid < n_ch) roff[tid] = incl - v;
        if (tid == 0) roff[n_ch] = tot;
        __syncthreads();
    }
    const uint32_t total = roff[n_ch];
    const uint32_t LB = (lbins && n_full > 0) ? lb_sh : 0u;
    const bool in_regs = total <= (uint32_t)kListWindow;

    // in registers: thread t holds entries u * 1024 + t (u < P), so that every
    // load instruction of a wave reads 512 consecutive bytes of a list
    uint64_t key[kListPer];
    const uint32_t P = in_regs ? (total + 1023) / 1024 : 0u;
    auto valid = [&](int u) { return (uint32_t)u < P && (uint32_t)u * 1024u + (uint32_t)tid < total; };
    if (in_regs) {
        // every entry's place in the lists first (no load is in flight while
        // this walks), as a 32-bit byte offset (a row's lists span at most
        // kListChunks * 4096 * 8 bytes), then all the loads at once
        int ch = 0;
        if ((uint32_t)tid < total) {
            int lo = 0, hi = n_ch;  // roff[lo] <= tid < roff[hi]
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (roff[mid] <= (uint32_t)tid) lo = mid; else hi = mid;
            }
            ch = lo;
        }
        uint32_t bound = roff[ch + 1], start = roff[ch];
        uint32_t at[kListPer];
#pragma unroll
        for (int u = 0; u < kListPer; ++u) {
            const uint32_t e = (uint32_t)u * 1024u + (uint32_t)tid;
            at[u] = 0;
            if (valid(u)) {
                while (e >= bound) {
                    ++ch;
                    start = bound;
                    bound = roff[ch + 1];
                }
                at[u] = 8u * ((uint32_t)ch * (uint32_t)chunk + (e - start));
            }
        }
        const char* lb = reinterpret_cast<const char*>(lrow);
#pragma unroll
        for (int u = 0; u < kListPer; ++u) key[u] = valid(u) ? *reinterpret_cast<const uint64_t*>(lb + at[u]) : 0ull;
    }
    // put(rank, u) for the register entries u whose bit is set in `take`,
    // ranked in list order (u, then wave, then lane): the count of every
    // (u, wave) pair, one block-wide scan over them, then the rank of each
    // entry from its pair's offset and the lanes below it.  Returns the total.
    auto rank_in_regs = [&](uint32_t take, auto&& put) {
#pragma unroll
        for (int u = 0; u < kListPer; ++u)
            if ((uint32_t)u < P) {
                const uint64_t m = __ballot((take >> u) & 1u);
                if (lane == 0) pcnt[16 * u + wave] = (uint32_t)__popcll(m);
            }
        __syncthreads();
        const uint32_t v = (uint32_t)tid < 16u * P ? pcnt[tid] : 0u;
        uint32_t tot;
        const uint32_t incl = block_scan_1024(v, wsum, &tot);
        if ((uint32_t)tid < 16u * P) pcnt[tid] = incl - v;
        __syncthreads();
        const uint64_t below = (1ull << lane) - 1;
#pragma unroll
        for (int u = 0; u < kListPer; ++u)
            if ((uint32_t)u < P) {
                const uint64_t m = __ballot((take >> u) & 1u);
                if ((take >> u) & 1u) put(pcnt[16 * u + wave] + (uint32_t)__popcll(m & below), u);
            }
        __syncthreads();  // pcnt is rewritten by the next call
        return tot;
    };
    // fn(key) for every list entry, in no particular order
    auto for_each_entry = [&](auto&& fn) {
        if (in_regs) {
#pragma unroll
            for (int u = 0; u < kListPer; ++u)
                if (valid(u)) fn(key[u]);
        } else {
            for (int ch = 0; ch < n_ch; ++ch) {
                const uint32_t cn = roff[ch + 1] - roff[ch];
                for (uint32_t j = tid; j < cn; j += 1024) fn(lrow[(int64_t)ch * chunk + j]);
            }
        }
    };
    // put(rank, key) for the entries with pick(key), ranked in list order,
    // streamed from memory; returns how many there are
    auto stream_ordered = [&](auto&& pick, auto&& put) {
        uint32_t base = 0;
        for (int ch = 0; ch < n_ch; ++ch) {
            const uint32_t cn = roff[ch + 1] - roff[ch];
            for (uint32_t j0 = 0; j0 < cn; j0 += 1024) {
                const uint32_t j = j0 + (uint32_t)tid;
                const uint64_t x = j < cn ? lrow[(int64_t)ch * chunk + j] : 0ull;
                const bool hit = j < cn && pick(x);
                const uint64_t m = __ballot(hit);
                if (lane == 0) wsum[wave] = (uint32_t)__popcll(m);
                __syncthreads();
                uint32_t off = base, tot = 0;
#pragma unroll
                for (int w2 = 0; w2 < 16; ++w2) {
                    off += w2 < wave ? wsum[w2] : 0u;
                    tot += wsum[w2];
                }
                if (hit) put(off + (uint32_t)__popcll(m & ((1ull << lane) - 1)), x);
                base += tot;
                __syncthreads();  // wsum is rewritten by the next step
            }
        }
        return base;
    };

    // 0. with the chunks' bound: the list entries at or above LB (a few times
    // K for distinct scores) go to LDS in any order, the K winners among
    // them are radix-selected on key64 from the top, marked in a bitmap by
    // position and written in position order.  More than kCandCap of them
    // (heavy ties) falls through to the search below.
    if (lbins) {
        if (in_regs) {
            uint32_t mask = 0;
#pragma unroll
            for (int u = 0; u < kListPer; ++u) mask |= (uint32_t)(valid(u) && key64_bin(key[u]) >= LB) << u;
            const uint32_t cnt = (uint32_t)__popc(mask);
            uint32_t incl = cnt;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const uint32_t u2 = __shfl_up(incl, o);
                if (lane >= o) incl += u2;
            }
            uint32_t base = 0;
            if (lane == 63 && incl) base = atomicAdd(&nsurv, incl);
            uint32_t off = __shfl(base, 63) + incl - cnt;
#pragma unroll
            for (int u = 0; u < kListPer; ++u)
                if ((mask >> u) & 1u) {
                    if (off < (uint32_t)kCandCap) c[off] = key[u];
                    ++off;
                }
        } else {
            for_each_entry([&](uint64_t x) {
                if (key64_bin(x) >= LB) {
                    const uint32_t r = atomicAdd(&nsurv, 1u);
                    if (r < (uint32_t)kCandCap) c[r] = x;
                }
            });
        }
        __syncthreads();
        const uint32_t n_surv = nsurv;
        if (n_surv <= (uint32_t)kCandCap) {
            select_in_lds(n_surv, false, false);
            return;
        }
    }

    // 1. the threshold bin B
    uint32_t B, above;
    find_bin([&](auto&& f) { for_each_entry([&](uint64_t x) { f(key64_bin(x)); }); }, kk, hcopy, dcount, thr,
             B, above);

    // 2. the entries at or above B, in order, into LDS while they fit
    uint32_t n_cand;
    if (in_regs) {
        uint32_t take = 0;
#pragma unroll
        for (int u = 0; u < kListPer; ++u) take |= (uint32_t)(valid(u) && key64_bin(key[u]) >= B) << u;
        n_cand = rank_in_regs(take, [&](uint32_t r, int u) {
            if (r < (uint32_t)kCandCap) c[r] = key[u];
        });
    } else {
        n_cand = stream_ordered([&](uint64_t x) { return key64_bin(x) >= B; },
                                [&](uint32_t r, uint64_t x) {
                                    if (r < (uint32_t)kCandCap) c[r] = x;
                                });
    }
    const bool in_lds = n_cand <= (uint32_t)kCandCap;
    if (tid == 0) {
        start_in_bin(&st, B, kk, above);
        st.done = 0;
    }
    __syncthreads();

    // 3. radix select among the threshold bin's keys
    while (!st.done) {
        if (tid < 256) hist256[tid] = 0;
        __syncthreads();
        const int sh = st.shift;
        const int w = digit_bits(sh);
        const uint64_t pf = st.prefix;
        auto count = [&](uint64_t x) {
            if (prefix_eq(x, sh, pf)) atomicAdd(&hist256[(uint32_t)(x >> (sh - w)) & ((1u << w) - 1u)], 1u);
        };
        if (in_lds) {
            for (uint32_t e = tid; e < n_cand; e += 1024) count(c[e]);
        } else {
            for_each_entry(count);  // entries below B never match the prefix
        }
        __syncthreads();
        radix_step(hist256, scan256, &st, &found);
    }
    const int sh = st.shift;
    const uint64_t pf = st.prefix;

    // 4. winners (key64 >= prefix << shift) in position order: per thread its
    // count, one block-wide scan, and each thread writes its run
    auto slot_of = [](uint64_t x) { return (int32_t)(0xFFFFFFFFu - (uint32_t)(x & 0xFFFFFFFFu)); };
    if (in_lds) {
        const uint32_t P2 = (n_cand + 1023) / 1024;  // <= kCandPer
        const uint32_t c_lo = P2 * (uint32_t)tid;
        uint32_t win = 0;
#pragma unroll
        for (int u = 0; u < kCandPer; ++u) {
            const uint32_t e = c_lo + (uint32_t)u;
            win |= (uint32_t)((uint32_t)u < P2 && e < n_cand && prefix_ge(c[e], sh, pf)) << u;
        }
        const uint32_t mine = (uint32_t)__popc(win);
        uint32_t tot;
        uint32_t p = block_scan_1024(mine, wsum, &tot) - mine;
#pragma unroll
        for (int u = 0; u < kCandPer; ++u)
            if ((win >> u) & 1u) {
                if (p < kk) out[p] = slot_of(c[c_lo + u]);
                ++p;
            }
    } else if (in_regs) {
        uint32_t win = 0;
#pragma unroll
        for (int u = 0; u < kListPer; ++u) win |= (uint32_t)(valid(u) && prefix_ge(key[u], sh, pf)) << u;
        rank_in_regs(win, [&](uint32_t r, int u) {
            if (r < kk) out[r] = slot_of(key[u]);
        });
    } else {
        stream_ordered([&](uint64_t x) { return prefix_ge(x, sh, pf); },
                       [&](uint32_t r, uint64_t x) {
                           if (r < kk) out[r] = slot_of(x);
                       });
    }
}

// The whole selection of a score row of at most kRowSelMax slots (Reindex
// pools, small block pools) in one workgroup of 1024 threads.  Thread t keeps
// the keys of slots t + 1024 u in registers; the threshold bin comes from
// find_bin, the keys of that bin are radix-selected from bit 51 down (the bins
// above it all win), the winners are marked in an LDS bitmap by slot and
// written in slot order (slot order is position order: a candidate list holds
// ascending positions, blocks are numbered by position).
constexpr int kRowPer = kRowSelMax / 1024;  // slots per thread

__global__ __launch_bounds__(1024) void k_topk_rows(const float* __restrict__ scores, int64_t stride, RowSrc rs,
                                                    const int32_t* __restrict__ cand, int cand_stride, int K,
                                                    int32_t* __restrict__ idx) {
    __shared__ uint32_t hcopy[64 * 32];
    __shared__ uint32_t dcount[64];
    __shared__ uint32_t hist256[256], scan256[256];
    __shared__ uint32_t bm[kRowSelMax / 32];
    __shared__ RadixState st;
    __shared__ int found;
    __shared__ uint32_t wsum[16];
    __shared__ uint32_t thr[2];
    const int row = blockIdx.x;
    const int tid = threadIdx.x;
    const float* sr = scores + (int64_t)row * stride;
    const int64_t n = row_n(rs, row);  // <= kRowSelMax (launcher)
    const uint32_t kk = (uint32_t)(n < K ? n : K);
    int32_t* out = idx + (int64_t)row * K;
    for (int i = tid + (int)kk; i < K; i += 1024) out[i] = -1;
    if (kk == 0) return;
    uint32_t key[kRowPer];
#pragma unroll
    for (int u = 0; u < kRowPer; ++u) {
        // unconditional loads (n >= 1 here; a slot past n re-reads slot n - 1
        // and every use checks valid(u)), so that they are issued together
        const int64_t e = tid + 1024 * u;
        key[u] = score_key(sr[e < n ? e : n - 1]);
    }
    auto valid = [&](int u) { return (int64_t)tid + 1024 * u < n; };
    if (tid == 0) {
        thr[0] = 0;
        thr[1] = 0;
    }
    if (tid < kRowSelMax / 32) bm[tid] = 0;
    __syncthreads();

    uint32_t B, above;
    find_bin(
        [&](auto&& f) {
#pragma unroll
            for (int u = 0; u < kRowPer; ++u)
                if (valid(u)) f(key_bin(key[u]));
        },
        kk, hcopy, dcount, thr, B, above);

    if (tid == 0) {
        start_in_bin(&st, B, kk, above);
        st.done = 0;
    }
    __syncthreads();
    while (!st.done) {
        if (tid < 256) hist256[tid] = 0;
        __syncthreads();
        const int sh = st.shift;
        const int w = digit_bits(sh);
        const uint64_t pf = st.prefix;
#pragma unroll
        for (int u = 0; u < kRowPer; ++u) {
            const uint64_t x = composite(key[u], (uint32_t)(tid + 1024 * u));
            if (valid(u) && prefix_eq(x, sh, pf)) atomicAdd(&hist256[(uint32_t)(x >> (sh - w)) & ((1u << w) - 1u)], 1u);
        }
        __syncthreads();
        radix_step(hist256, scan256, &st, &found);
    }
    const int sh = st.shift;
    const uint64_t pf = st.prefix;
#pragma unroll
    for (int u = 0; u < kRowPer; ++u) {
        const uint32_t e = (uint32_t)(tid + 1024 * u);
        if (valid(u) && prefix_ge(composite(key[u], e), sh, pf)) atomicOr(&bm[e >> 5], 1u << (e & 31));
    }
    __syncthreads();
    // slots in order: thread t owns bitmap word t
    const int nwords = (int)((n + 31) / 32);
    uint32_t wd = tid < nwords ? bm[tid] : 0u;
    const uint32_t cnt = (uint32_t)__popc(wd);
    uint32_t tot;
    uint32_t r = block_scan_1024(cnt, wsum, &tot) - cnt;
    while (wd) {
        const int bit = __ffs(wd) - 1;
        const uint32_t slot = 32u * (uint32_t)tid + (uint32_t)bit;
        if (r < kk) out[r] = map_slot(cand, cand_stride, row, slot);
        ++r;
        wd &= wd - 1;
    }
}

// ---------------------------------------------------------------------------
// block pool
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_block_max(const float* __restrict__ scores, int64_t stride, RowSrc rs,
                                                   float* __restrict__ bscores, int64_t bstride) {
    const int row = blockIdx.y;
    const int b = rs.row_seq[row];
    const int64_t n = rs.entry_off[b + 1] - rs.entry_off[b];
    const int64_t vis = visible_count(n, rs.q_pos[row], rs.ratio);
    const int64_t nb = (vis + rs.block - 1) / rs.block;
    const int64_t blk = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (blk >= nb) return;
    const float* sr = scores + (int64_t)row * stride;
    float m = -INFINITY;
    for (int64_t j = blk * rs.block; j < (blk + 1) * rs.block && j < vis; ++j) m = fmaxf(m, sr[j]);
    bscores[(int64_t)row * bstride + blk] = m;
}

__global__ __launch_bounds__(256) void k_pool_expand(const int32_t* __restrict__ blocks, RowSrc rs, int max_blocks,
                                                     int32_t* __restrict__ pool_pos, int32_t* __restrict__ pool_count) {
    __shared__ uint32_t part[256];
    const int row = blockIdx.x;
    const int b = rs.row_seq[row];
    const int64_t n = rs.entry_off[b + 1] - rs.entry_off[b];
    const int64_t vis = visible_count(n, rs.q_pos[row], rs.ratio);
    const int32_t* br = blocks + (int64_t)row * max_blocks;
    int32_t* pr = pool_pos + (int64_t)row * max_blocks * rs.block;
    const int per = (max_blocks + 255) / 256;  // blocks per thread, in order
    const int t = threadIdx.x;
    uint32_t mine = 0;
    for (int i = t * per; i < (t + 1) * per && i < max_blocks; ++i) {
        const int32_t bb = br[i];
        if (bb >= 0) {
            const int64_t lo = (int64_t)bb * rs.block;
            const int64_t hi = lo + rs.block < vis ? lo + rs.block : vis;
            mine += (uint32_t)(hi > lo ? hi - lo : 0);
        }
    }
    part[t] = mine;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
        const uint32_t v = t >= off ? part[t - off] : 0;
        __syncthreads();
        part[t] += v;
        __syncthreads();
    }
    uint32_t w = part[t] - mine;
    for (int i = t * per; i < (t + 1) * per && i < max_blocks; ++i) {
        const int32_t bb = br[i];
        if (bb >= 0) {
            const int64_t lo = (int64_t)bb * rs.block;
            const int64_t hi = lo + rs.block < vis ? lo + rs.block : vis;
            for (int64_t j = lo; j < hi; ++j) pr[w++] = (int32_t)j;
        }
    }
    const uint32_t total = part[255];
    for (int64_t i = total + t; i < (int64_t)max_blocks * rs.block; i += 256) pr[i] = -1;
    if (t == 0) pool_count[row] = (int32_t)total;
}

size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

size_t topk_ws_bytes(int total_q) {
    return al256((size_t)total_q * kHistBins * 4) + al256((size_t)total_q * sizeof(RowSel)) +
           al256((size_t)total_q * kCandCap * 8);
}

uint32_t* topk_ws_hist(void* ws) { return (uint32_t*)ws; }

hipError_t clear_topk_ws(void* ws, int nq, bool hist_too, hipStream_t s) {
    // histogram and row state are adjacent: clear both with one fill
    const size_t hb = al256((size_t)nq * kHistBins * 4);
    char* base = (char*)ws + (hist_too ? 0 : hb);
    const int64_t nfill = (int64_t)(((hist_too ? hb : 0) + al256((size_t)nq * sizeof(RowSel))) / 4);
    hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)((nfill + 255) / 256 < 2048 ? (nfill + 255) / 256 : 2048)), dim3(256), 0,
                       s, (uint32_t*)base, nfill, 0u);
    return hipGetLastError();
}

hipError_t launch_topk(const TopkLaunch& a, hipStream_t s) {
    const int nq = a.g.total_q;
    char* ws = (char*)a.ws;
    uint32_t* hist = (uint32_t*)ws;
    ws += al256((size_t)nq * kHistBins * 4);
    RowSel* sel = (RowSel*)ws;
    ws += al256((size_t)nq * sizeof(RowSel));
    uint64_t* cb = (uint64_t*)ws;
    RowSrc rs{a.b->d_entry_off, a.b->d_row_seq, a.b->d_q_pos, a.b->ratio, a.cand ? a.cand_count : nullptr,
              a.block_mode, a.block, a.max_slots};
    if (a.max_slots <= kRowSelMax) {  // one workgroup per row; any histogram from the caller is not needed
        hipLaunchKernelGGL(k_topk_rows, dim3(nq), dim3(1024), 0, s, a.scores, a.stride, rs, a.cand, a.cand_stride,
                           a.K, a.idx);
        return hipGetLastError();
    }
    const unsigned chunks = (unsigned)((a.max_slots + kHChunk - 1) / kHChunk);
    const uint32_t* h = a.hist;
    if (!h) {
        // no histogram from the caller: the chunk bounds (in the histogram's
        // place) give a lower bound of each row's threshold bin
        hipError_t e = clear_topk_ws(a.ws, nq, false, s);
        if (e != hipSuccess) return e;
        // with the scorer's tile maxima, rows of at least K tiles take the
        // tile bound and skip the chunk bounds
        const uint32_t* tb = nullptr;
        if (a.tmax && a.tb) {
            hipLaunchKernelGGL(k_tile_bound, dim3(nq), dim3(256), 0, s, a.tmax, a.tstride, rs, a.K, a.tb);
            tb = a.tb;
        }
        const int cs = bound_stride(a.K);
        const unsigned sampled = (chunks + cs - 1) / cs;
        hipLaunchKernelGGL(k_chunk_bound, dim3(sampled ? sampled : 1, nq), dim3(256), 0, s, a.scores, a.stride, rs, a.K,
                           cs, tb, hist);
        hipLaunchKernelGGL(k_collect<true>, dim3(chunks ? chunks : 1, nq), dim3(256), 0, s, a.scores, a.stride, rs,
                           hist, a.K, cs, a.tmax, a.tstride, tb, sel, cb);
    } else {
        if (h != hist) {
            hipError_t e = clear_topk_ws(a.ws, nq, false, s);
            if (e != hipSuccess) return e;
        }
        // (h == hist: the caller cleared the workspace and filled its histogram)
        hipLaunchKernelGGL(k_collect<false>, dim3(chunks ? chunks : 1, nq), dim3(256), 0, s, a.scores, a.stride, rs, h,
                           a.K, 1, (const uint32_t*)nullptr, (int64_t)0, (const uint32_t*)nullptr, sel, cb);
    }
    hipLaunchKernelGGL(k_final, dim3(nq), dim3(1024), 0, s, a.scores, a.stride, sel, cb, a.cand, a.cand_stride, a.K,
                       a.idx);
    return hipGetLastError();
}

hipError_t launch_topk_local(const csa2_batch* b, const Geometry& g, const LocalOut& lo, int32_t* idx, void* ws,
                             hipStream_t s) {
    const int nq = g.total_q;
    const uint32_t* hist = (const uint32_t*)ws;
    RowSel* sel = (RowSel*)((char*)ws + al256((size_t)nq * kHistBins * 4));
    RowSrc rs{b->d_entry_off, b->d_row_seq, b->d_q_pos, b->ratio, nullptr, 0, 1, g.max_entries};
    hipLaunchKernelGGL(k_row_threshold, dim3(nq), dim3(256), 0, s, hist, rs, lo.K, sel);
    hipLaunchKernelGGL(k_collect_local, dim3((unsigned)lo.max_chunks, nq), dim3(256), 0, s, lo.lists, lo.counts,
                       lo.max_chunks, lo.chunk, (const RowSel*)sel);
    hipLaunchKernelGGL(k_final_local, dim3(nq), dim3(1024), 0, s, (const uint64_t*)lo.lists, (const uint32_t*)lo.counts,
                       lo.max_chunks, lo.chunk, (const RowSel*)sel, lo.K, idx);
    return hipGetLastError();
}

hipError_t launch_topk_fused(const csa2_batch* b, const Geometry& g, const LocalOut& lo, int32_t* idx, void* ws,
                             hipStream_t s) {
    if (lo.max_chunks > kListChunks || (int64_t)lo.max_chunks * lo.chunk > kFusedTopkEntries ||
        lo.chunk < 256 * kSpecPer || lo.max_chunks > kPartChunks * kMaxParts)
        return hipErrorInvalidValue;
    RowSrc rs{b->d_entry_off, b->d_row_seq, b->d_q_pos, b->ratio, nullptr, 0, 1, g.max_entries};
    const int nq = g.total_q;
    // with the chunks' bounds: the parts' counts in the workspace's histogram
    // area, their entries in its candidate area (kCandCap per row)
    uint32_t* part_cnt = nullptr;
    uint32_t* part_n = nullptr;
    uint64_t* part_keys = nullptr;
    int parts = 0, cap = 0;
    if (lo.lbins && ws) {
        parts = (lo.max_chunks + kPartChunks - 1) / kPartChunks;  // <= kMaxParts (checked above)
        cap = kCandCap / parts;
        part_cnt = (uint32_t*)ws;  // [nq][parts], then [nq] sizes: within the histogram area
        part_n = part_cnt + (size_t)nq * parts;
        part_keys = (uint64_t*)((char*)ws + al256((size_t)nq * kHistBins * 4) + al256((size_t)nq * sizeof(RowSel)));
        hipLaunchKernelGGL(k_lists_filter, dim3(parts, nq), dim3(256), 0, s, (const uint64_t*)lo.lists,
                           (const uint32_t*)lo.counts, (const uint32_t*)lo.lbins, lo.max_chunks, lo.chunk, rs, cap,
                           part_cnt, part_n, part_keys);
    }
    hipLaunchKernelGGL(k_topk_lists, dim3(nq), dim3(1024), 0, s, (const uint64_t*)lo.lists, (const uint32_t*)lo.counts,
                       (const uint32_t*)lo.lbins, lo.max_chunks, lo.chunk, rs, lo.K, (const uint32_t*)part_cnt,
                       (const uint32_t*)part_n, (const uint64_t*)part_keys, parts, cap, idx);
    return hipGetLastError();
}

hipError_t launch_block_pool(const PoolLaunch& a, hipStream_t s) {
    RowSrc rs{a.b->d_entry_off, a.b->d_row_seq, a.b->d_q_pos, a.b->ratio, nullptr, 1, a.block,
              (a.g.max_entries + a.block - 1) / a.block};
    const int64_t max_nb = (a.g.max_entries + a.block - 1) / a.block;
    if (!a.bscores_ready)
        hipLaunchKernelGGL(k_block_max, dim3((unsigned)((max_nb + 255) / 256), a.g.total_q), dim3(256), 0, s, a.scores,
                           a.stride, rs, a.bscores, a.bstride);
    TopkLaunch t{};
    t.b = a.b;
    t.g = a.g;
    t.scores = a.bscores;
    t.stride = a.bstride;
    t.max_slots = max_nb;
    t.cand = nullptr;
    t.cand_stride = 0;
    t.cand_count = nullptr;
    t.block_mode = 1;
    t.block = a.block;
    t.K = a.max_blocks;
    t.idx = a.blocks;
    t.ws = a.topk_ws;
    t.hist = nullptr;
    hipError_t e = launch_topk(t, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_pool_expand, dim3(a.g.total_q), dim3(256), 0, s, a.blocks, rs, a.max_blocks, a.pool_pos,
                       a.pool_count);
    return hipGetLastError();
}

}  // namespace csa2
