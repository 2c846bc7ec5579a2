// Gather + dequantise of the selected main-KV latents, and sparse latent
// attention over [selected entries ++ SWA window].
//
// Report "DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache Compression":
// section 2.3 (each query attends to its Top-K entries together with the
// layer-local sliding-window KV), section 2.4.4 (FP4 main KV is dequantised
// before attention), section 4.2.1 (64 query heads of dim 512 sharing one
// latent, window 128).  The reading note "DeepSeek V4.1 Flash: Pushing the
// Limits of KV Cache Compression" (Figure 4 reading) has the selected main KV
// concatenated with the SWA KV and handed to core attention as one key set.
// Course notes "3. 通用基础设施", section 3.2.2: query i sees SWA keys
// [max(s, i-W+1), i].
//
// The dequantised bf16 latents are exact (attn_common.h).
#include "attn_common.h"

namespace csa2 {
namespace {

using namespace attn;

// ---------------------------------------------------------------------------
// gather + dequantise: grid (K, total_q), 64 threads, 8 channels per thread
// ---------------------------------------------------------------------------
template <int KVF>
__global__ __launch_bounds__(64) void k_gather_dequant(const uint8_t* __restrict__ kv, const uint8_t* __restrict__ kv_sc,
                                                       const int64_t* __restrict__ entry_off,
                                                       const int32_t* __restrict__ row_seq,
                                                       const int32_t* __restrict__ idx, int K,
                                                       uint16_t* __restrict__ out) {
    const int s = blockIdx.x, row = blockIdx.y, t = threadIdx.x;
    const int32_t j = idx[(int64_t)row * K + s];
    const int b = row_seq[row];
    v4i v = {0, 0, 0, 0};
    if (j >= 0 && j < entry_off[b + 1] - entry_off[b]) {  // out-of-range entries read as empty
        const int64_t e = entry_off[b] + j;
        const uint32_t codes = *reinterpret_cast<const uint32_t*>(kv + e * 256 + 4 * t);
        if constexpr (KVF == kKvE4)
            v = fp4x8_to_bf16_mul(codes, e4m3_f32(kv_sc[e * 32 + (8 * t) / 16]));
        else
            v = fp4x8_to_bf16(codes, e8m0_f32(kv_sc[e * 16 + (8 * t) / 32]));
    }
    *reinterpret_cast<v4i*>(out + ((int64_t)row * K + s) * 512 + 8 * t) = v;
}

// ---------------------------------------------------------------------------
// sparse attention: one workgroup per (query row, group of 16 heads), NP
// groups of 4 waves ("pipes").  Keys come in blocks of 64: first the SWA rows
// of the window, then the selected entries (idx order); pipe g takes the
// blocks blk0 + NP i + g of its part of the row, each pipe with its own LDS
// key buffer and its own online-softmax state.  Per block: dequantise into
// LDS (row-major bf16), S = Q K^T on v_mfma_f32_16x16x32_bf16 (wave w: keys
// 16w..16w+15), online softmax in fp32, O += P V (wave w: channels
// 128w..128w+127) with V read transposed by ds_read_b64_tr_b16.  With two
// pipes their (max, sums, O) are merged at the end.  The loads of the first
// iteration (the SWA rows) are issued together with the query and the index
// row; later blocks are fetched one iteration ahead.  The waves share data
// through LDS only, so their barriers order LDS only and leave the prefetch
// in flight.  One pipe keeps the LDS of a workgroup at 73 KB, so that two
// workgroups share a CU; measured, that
// beats two pipes in one workgroup except on the smallest grids.
// ---------------------------------------------------------------------------
constexpr int HG = 16;
constexpr int SLROW = KB + 4;  // LDS row stride of the logits in floats

template <int NPIPE, int KVF, int SWF, int ROPE>
__global__ __launch_bounds__(256 * NPIPE) void k_sparse_attn(
    const uint16_t* __restrict__ q, int Hm, const uint8_t* __restrict__ kv, const uint8_t* __restrict__ kv_sc,
    const int32_t* __restrict__ idx, int K, const void* __restrict__ swa, const int64_t* __restrict__ swa_row_off,
    const int32_t* __restrict__ swa_pos0, const int32_t* __restrict__ replay_s, int W,
    const int64_t* __restrict__ entry_off, const int32_t* __restrict__ row_seq, const int32_t* __restrict__ q_pos,
    float scale_log2, void* __restrict__ out, float* __restrict__ lse, int total_q, int n_hg, int S,
    float* __restrict__ partial, const float* __restrict__ rope_cs) {
    __shared__ __attribute__((aligned(16))) uint16_t kl[NPIPE][KB * LROW];
    __shared__ float sl[NPIPE][HG][SLROW];
    __shared__ int kvalid[NPIPE][KB];
    __shared__ int32_t kidx[kMaxK];
    __shared__ float mls[HG][3];
    __shared__ int nsel_sh;

    // the n_hg x S workgroups of one row share an XCD (workgroups are dealt to
    // XCDs round-robin), so the row's gathered keys are read from one L2
    const int L = blockIdx.x;
    const int xcd = L & 7;
    const int kq = L >> 3;
    const int units = n_hg * S;
    const int hg = (kq % units) / S;
    const int sp = (kq % units) % S;  // which part of the row's key blocks
    const int row = (kq / units) * 8 + xcd;
    if (row >= total_q) return;

    const int tid = threadIdx.x;
    const int pipe = NPIPE == 1 ? 0 : __builtin_amdgcn_readfirstlane(tid >> 8);
    const int pt = tid & 255;  // thread within the pipe
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane((tid >> 6) & 3);  // wave within the pipe
    const int lg = lane >> 4, li = lane & 15;

    // ---- prologue: the index row and the query first (they need only the
    // row), then the sequence's window and, with it, the first block's SWA rows.
    // The index row goes first: loads complete in issue order, and the index
    // row is needed first (in LDS, before any selected key is fetched), so its
    // wait leaves the query's 16 KB in flight.
    const int32_t* irow = idx + (int64_t)row * K;
    constexpr int NT = 256 * NPIPE;
    int32_t ir[kMaxK / NT];
#pragma unroll
    for (int i = 0; i < kMaxK / NT; ++i) {
        const int s = tid + NT * i;
        ir[i] = s < K ? irow[s] : -1;
    }
    __builtin_amdgcn_sched_barrier(0);  // keeps the index row's loads ahead of the query's
    const int hq = HG * hg + li;
    v8bf Q[16];
    const float* row_cs = ROPE ? rope_cs + (int64_t)row * 64 : nullptr;
    {
        const int64_t qr = ((int64_t)row * Hm + hq) * 512 + 8 * lg;
        load_q16<ROPE>(Q, q, qr, lg, row_cs);
    }
    // keep the loads above ahead of the scalar loads below (they would
    // otherwise wait for them)
    asm volatile("" ::: "memory");

    const int b = row_seq[row];
    const int64_t t = q_pos[row];
    const int64_t e0 = entry_off[b];
    const int64_t n_ent = entry_off[b + 1] - e0;
    const int64_t s_rep = replay_s ? (int64_t)replay_s[b] : 0;
    int64_t u_lo = t - W + 1;
    u_lo = u_lo > s_rep ? u_lo : s_rep;
    const int n_swa = t >= u_lo ? (int)(t - u_lo + 1) : 0;
    const int64_t swa_r0 = swa_row_off[b] + (u_lo - swa_pos0[b]);  // row of key 0 in `swa`

    // the split of the row's blocks over the S workgroups is fixed by the
    // largest key count (window + K), so it is known before the index row
    const int max_blocks = (n_swa + K + KB - 1) / KB;
    const int per = (max_blocks + S - 1) / S;
    const int blk0 = sp * per;
    const int blk1 = blk0 + per < max_blocks ? blk0 + per : max_blocks;
    const int n_it = (blk1 - blk0 + NPIPE - 1) / NPIPE;

    // this thread stages key `skey` of its pipe's blocks, channels CP*part .. +CP
    constexpr int CP = 128;         // channels per part (4 parts)
    constexpr int NB = CP / 32;     // 32-channel scale blocks per part
    const int skey = (pt & 15) + 16 * (pt >> 6), part = (pt >> 4) & 3;

    const int vk_first = KB * (blk0 + pipe) + skey;
    const bool first_swa = blk0 + pipe < blk1 && vk_first < n_swa;
    // this thread's 128 channels of SWA row vk: 16 bf16 loads, or 8 loads of
    // MXFP8 codes and one of their 4 scales
    v4i sw[CP / 8];
    uint32_t swsc = 0;
    auto load_swa = [&](int vk) {
        if constexpr (SWF == kSwaMx8) {
            const uint8_t* rb = reinterpret_cast<const uint8_t*>(swa) + (swa_r0 + vk) * 528;
#pragma unroll
            for (int i = 0; i < CP / 16; ++i) sw[i] = ld16(rb + CP * part + 16 * i);
            swsc = *reinterpret_cast<const uint32_t*>(rb + 512 + 4 * part);
        } else {
            const uint16_t* src = reinterpret_cast<const uint16_t*>(swa) + (swa_r0 + vk) * 512 + CP * part;
#pragma unroll
            for (int i = 0; i < CP / 8; ++i) sw[i] = ld16(src + 8 * i);
        }
    };
    if (first_swa) load_swa(vk_first);
    if (tid == 0) nsel_sh = 0;
    lds_barrier();
    {
        int last = 0;
#pragma unroll
        for (int i = 0; i < kMaxK / NT; ++i) {
            const int s = tid + NT * i;
            if (s < K) {
                const int32_t j = (ir[i] >= 0 && ir[i] < n_ent) ? ir[i] : -1;  // out-of-range entries read as empty
                kidx[s] = j;
                if (j >= 0) last = s + 1;
            }
        }
        if (last) atomicMax(&nsel_sh, last);
    }
    lds_barrier();
    const int n_sel = nsel_sh;
    const int n_keys = n_swa + n_sel;

    v4f O[8];
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) O[nt] = v4f{0.f, 0.f, 0.f, 0.f};
    // running max and sums for head li (identical in every wave of a pipe):
    // l_run sums the bf16 weights the P V product uses (it normalises the
    // output), l_lse the fp32 weights (it gives the log-sum-exp)
    float m_run = -INFINITY, l_run = 0.0f, l_lse = 0.0f;

    // FP4 rows of a selected key, fetched one iteration ahead, with their
    // scales: 4 E8M0 (one per 32 channels) or 8 E4M3 (one per 16 channels)
    v4i pc[NB];
    uint32_t psc = 0, psc2 = 0;
    auto fetch = [&](int blk) {
        const int vk = KB * blk + skey;
        if (blk < blk1 && vk >= n_swa && vk < n_keys) {
            const int32_t j = kidx[vk - n_swa];
            if (j >= 0) {
                const int64_t e = e0 + j;
                const uint8_t* src = kv + e * 256 + (CP / 2) * part;
#pragma unroll
                for (int i = 0; i < NB; ++i) pc[i] = ld16(src + 16 * i);
                if constexpr (KVF == kKvE4) {
                    const uint2 w2 = *reinterpret_cast<const uint2*>(kv_sc + e * 32 + 8 * part);
                    psc = w2.x;
                    psc2 = w2.y;
                } else {
                    psc = *reinterpret_cast<const uint32_t*>(kv_sc + e * 16 + 4 * part);
                }
            }
        }
    };
    // stage this thread's key of block blk into the pipe's buffer: SWA rows
    // from `sw` (first iteration) or loaded here (windows longer than the
    // first iteration's blocks), selected entries from the prefetched FP4 rows
    uint16_t* klp = kl[pipe];
    auto stage = [&](int blk, bool swa_in_regs) {
        const int vk = KB * blk + skey;
        uint16_t* dst = klp + skey * LROW + CP * part;
        int valid = 0;
        if (vk < n_swa) {
            valid = 1;
            if (!swa_in_regs) load_swa(vk);
            if constexpr (SWF == kSwaMx8) {
                // E4M3 x E8M0 is exact in bf16 (four significant bits, a power of two)
#pragma unroll
                for (int i = 0; i < NB; ++i) {  // 32 channels per scale
                    const float sc = e8m0_f32((swsc >> (8 * i)) & 255u);
#pragma unroll
                    for (int d = 0; d < 4; ++d) {  // 8 channels: two dwords of 4 codes
                        const uint32_t w0 = (uint32_t)sw[2 * i + d / 2][2 * (d % 2)];
                        const uint32_t w1 = (uint32_t)sw[2 * i + d / 2][2 * (d % 2) + 1];
                        auto a0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, sc, false);
                        auto a1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, sc, true);
                        auto b0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, sc, false);
                        auto b1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, sc, true);
                        *reinterpret_cast<v8bf*>(dst + 32 * i + 8 * d) =
                            v8bf{a0[0], a0[1], a1[0], a1[1], b0[0], b0[1], b1[0], b1[1]};
                    }
                }
            } else {
#pragma unroll
                for (int i = 0; i < CP / 8; ++i) *reinterpret_cast<v4i*>(dst + 8 * i) = sw[i];
            }
        } else if (vk < n_keys && kidx[vk - n_swa] >= 0) {
            valid = 1;
#pragma unroll
            for (int i = 0; i < NB; ++i) {  // 32 channels
                if constexpr (KVF == kKvE4) {  // a scale per 16 channels: bytes 2i, 2i + 1 of psc:psc2
                    const uint32_t w = i < 2 ? psc : psc2;
                    const float s0 = e4m3_f32((w >> (16 * (i & 1))) & 255u);
                    const float s1 = e4m3_f32((w >> (16 * (i & 1) + 8)) & 255u);
#pragma unroll
                    for (int d = 0; d < 4; ++d)
                        *reinterpret_cast<v4i*>(dst + 32 * i + 8 * d) =
                            fp4x8_to_bf16_mul((uint32_t)pc[i][d], d < 2 ? s0 : s1);
                } else {
                    const float sc = e8m0_f32((psc >> (8 * i)) & 255u);
#pragma unroll
                    for (int d = 0; d < 4; ++d)
                        *reinterpret_cast<v4i*>(dst + 32 * i + 8 * d) = fp4x8_to_bf16((uint32_t)pc[i][d], sc);
                }
            }
        }
        if (!valid) {
#pragma unroll
            for (int i = 0; i < CP / 8; ++i) *reinterpret_cast<v4i*>(dst + 8 * i) = v4i{0, 0, 0, 0};
        }
        if (part == 0) kvalid[pipe][skey] = valid;
    };

    // first iteration: a selected key in it is loaded now (short windows or a
    // later part of the row); the next iteration's rows are fetched behind it
    if (blk0 + pipe < blk1) {
        fetch(blk0 + pipe);
        stage(blk0 + pipe, true);
    }
    fetch(blk0 + pipe + NPIPE);

    for (int it = 0; it < n_it; ++it) {
        const int blk = blk0 + NPIPE * it + pipe;
        const bool active = blk < blk1 && KB * blk < n_keys;  // uniform per pipe
        if (it > 0) {
            if (blk < blk1) stage(blk, false);
            fetch(blk + NPIPE);
        }
        lds_barrier();

        // 2) S = Q K^T for keys 16*wave .. +16: lane gets S[head 4lg+v][key 16wave + li]
        if (active) {
            // four independent accumulation chains over the 16 k-steps
            v4f Sp[4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
            const uint16_t* kr = klp + (16 * wave + li) * LROW + 8 * lg;
#pragma unroll
            for (int ks = 0; ks < 16; ++ks) {
                const v8bf Bk = __builtin_bit_cast(v8bf, *reinterpret_cast<const v4i*>(kr + 32 * ks));
                Sp[ks & 3] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Q[ks], Bk, Sp[ks & 3], 0, 0, 0);
            }
            const v4f Sv = (Sp[0] + Sp[1]) + (Sp[2] + Sp[3]);
            const int key = 16 * wave + li;
            const bool ok = kvalid[pipe][key] != 0;
#pragma unroll
            for (int v = 0; v < 4; ++v) sl[pipe][4 * lg + v][key] = ok ? Sv[v] * scale_log2 : -INFINITY;
        }
        lds_barrier();

        if (active) {
            // 3) online softmax (base 2) for head li over keys 8lg + 32ks + i
            float p[16];
            float mx = -INFINITY;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    p[8 * ks + i] = sl[pipe][li][8 * lg + 32 * ks + i];
                    mx = fmaxf(mx, p[8 * ks + i]);
                }
            mx = xor_max<16>(mx);
            mx = xor_max<32>(mx);
            const float m_new = fmaxf(m_run, mx);
            float alpha;
            // each weight as the sum of two bf16 values (hi + lo), so that the P V
            // product carries about 16 significant bits of it; a single bf16 weight
            // (8 bits) costs up to ~3e-3 of absolute output error when a handful of
            // keys carry the softmax
            v8bf P[2], Plo[2];
            float rs = 0.0f, rs32 = 0.0f;
            if (m_new == -INFINITY) {  // nothing valid yet
                alpha = 1.0f;
#pragma unroll
                for (int i = 0; i < 16; ++i) p[i] = 0.0f;
            } else {
                // arguments are <= 0 (or -inf): the plain hardware exp2, whose
                // flush of results below 2^-126 to zero is immaterial here
                alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // m_run = -inf -> 0
#pragma unroll
                for (int i = 0; i < 16; ++i) p[i] = __builtin_amdgcn_exp2f(p[i] - m_new);
            }
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const __bf16 pb = (__bf16)p[8 * ks + i];
                    const __bf16 pl = (__bf16)(p[8 * ks + i] - (float)pb);
                    P[ks][i] = pb;
                    Plo[ks][i] = pl;
                    rs += (float)pb + (float)pl;  // normalise with the weights actually used
                    rs32 += p[8 * ks + i];
                }
            rs = xor_sum<16>(rs);
            rs = xor_sum<32>(rs);
            rs32 = xor_sum<16>(rs32);
            rs32 = xor_sum<32>(rs32);
            l_run = l_run * alpha + rs;
            l_lse = l_lse * alpha + rs32;
            m_run = m_new;
            // O rows are heads 4lg + v: fetch their alpha from lane (4lg + v)
            float av[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) av[v] = __shfl(alpha, 4 * lg + v);
#pragma unroll
            for (int nt = 0; nt < 8; ++nt)
#pragma unroll
                for (int v = 0; v < 4; ++v) O[nt][v] *= av[v];

            // 4) O += P V for channels 128*wave + 16nt + li
#pragma unroll
            for (int nt = 0; nt < 8; ++nt) {
                const int n0 = 128 * wave + 16 * nt;
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const int kb = 8 * lg + 32 * ks;
                    const uint16_t* a0 = klp + (kb + (li >> 2)) * LROW + n0 + 4 * (li & 3);
                    const uint16_t* a1 = klp + (kb + 4 + (li >> 2)) * LROW + n0 + 4 * (li & 3);
                    const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(a0));
                    const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(a1));
                    const v8s both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                    const v8bf vb = __builtin_bit_cast(v8bf, both);
                    O[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(P[ks], vb, O[nt], 0, 0, 0);
                    O[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Plo[ks], vb, O[nt], 0, 0, 0);
                }
            }
        }
        lds_barrier();
    }

    // merge the pipes: pipe 1 leaves its state in LDS (its key buffer), pipe 0
    // combines: with M = max(m0, m1) and a_g = 2^(m_g - M), O = a0 O0 + a1 O1
    if constexpr (NPIPE == 2) {
        float* ob = reinterpret_cast<float*>(kl[1]);  // 16 x 512 floats
        if (pipe == 1) {
#pragma unroll
            for (int nt = 0; nt < 8; ++nt)
#pragma unroll
                for (int v = 0; v < 4; ++v) ob[(4 * lg + v) * 512 + 128 * wave + 16 * nt + li] = O[nt][v];
            if (wave == 0 && lane < 16) {
                mls[lane][0] = m_run;
                mls[lane][1] = l_run;
                mls[lane][2] = l_lse;
            }
        }
        lds_barrier();
        if (pipe == 1) return;
        {
            const float m1 = mls[li][0];
            const float M = fmaxf(m_run, m1);
            const float a0 = M == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run - M);
            const float a1 = M == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m1 - M);
            l_run = a0 * l_run + a1 * mls[li][1];
            l_lse = a0 * l_lse + a1 * mls[li][2];
            m_run = M;
            float b0[4], b1[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                b0[v] = __shfl(a0, 4 * lg + v);
                b1[v] = __shfl(a1, 4 * lg + v);
            }
#pragma unroll
            for (int nt = 0; nt < 8; ++nt)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    O[nt][v] = b0[v] * O[nt][v] + b1[v] * ob[(4 * lg + v) * 512 + 128 * wave + 16 * nt + li];
        }
        }

    if (S > 1) {
        // partial result of this part of the keys: unnormalised O, its max and
        // both sums, combined by k_attn_combine
        float* po = partial + (((int64_t)row * n_hg + hg) * S + sp) * (HG * 516);
#pragma unroll
        for (int nt = 0; nt < 8; ++nt)
#pragma unroll
            for (int v = 0; v < 4; ++v) po[(4 * lg + v) * 512 + 128 * wave + 16 * nt + li] = O[nt][v];
        if (wave == 0 && lane < 16) {
            po[HG * 512 + 4 * lane + 0] = m_run;
            po[HG * 512 + 4 * lane + 1] = l_run;
            po[HG * 512 + 4 * lane + 2] = l_lse;
        }
        return;
    }
    // finalise: O / l for heads 4lg + v
    const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;
    float iv[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) iv[v] = __shfl(inv, 4 * lg + v);
    // channel 128 wave + 16 nt + li is in the rotated part in wave 3 from nt = 4 on
    float2 ang[4] = {};
    if constexpr (ROPE)
        if (wave == 3) load_out_angles(ang, row_cs, li);
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
#pragma unroll
        for (int v = 0; v < 4; ++v)
            store_out<ROPE>(out, ((int64_t)row * Hm + HG * hg + 4 * lg + v) * 512 + 128 * wave + 16 * nt + li,
                            128 * wave + 16 * nt + li, O[nt][v] * iv[v], wave == 3 && nt >= 4,
                            ang[nt >= 4 ? nt - 4 : 0]);
    if (lse && wave == 0 && lane < 16)
        lse[(int64_t)row * Hm + HG * hg + lane] =
            l_lse > 0.0f ? (m_run + log2f(l_lse)) * 0.69314718055994531f : -INFINITY;
}

// Merge the S partial results of each (row, head): with M = max_s m_s and
// a_s = 2^(m_s - M), O = sum_s a_s O_s / sum_s a_s l_s.  One workgroup of 128
// threads per (row, head); thread t owns channels 4t .. 4t+3, so every load of
// the merge is issued at once.
constexpr int kMaxSplit = 8;  // the combine is instantiated for S = 2 .. kMaxSplit
constexpr int kAttnTargetWgs = 256;  // workgroups the key splits aim for (more splits cost more than they hide)
constexpr unsigned kAttnTwoPipeWgs = 128;  // grids up to this size run two pipes per workgroup

template <int S, int ROPE>
__global__ __launch_bounds__(128) void k_attn_combine(const float* __restrict__ part, int Hm, int n_hg,
                                                      void* __restrict__ out, float* __restrict__ lse,
                                                      const float* __restrict__ rope_cs) {
    const int row = blockIdx.x / Hm, h = blockIdx.x % Hm;
    const int hg = h / HG, hh = h % HG;
    const float* base = part + ((int64_t)row * n_hg + hg) * S * (HG * 516);
    const int t = threadIdx.x;
    float m[S], l[S], ll[S];
    v4f o[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const float* ps = base + s * (HG * 516);
        m[s] = ps[HG * 512 + 4 * hh];  // the same address in every lane: one scalar load
        l[s] = ps[HG * 512 + 4 * hh + 1];
        ll[s] = ps[HG * 512 + 4 * hh + 2];
        o[s] = *reinterpret_cast<const v4f*>(ps + hh * 512 + 4 * t);
    }
    float M = -INFINITY;
#pragma unroll
    for (int s = 0; s < S; ++s) M = fmaxf(M, m[s]);
    float L = 0.0f, Llse = 0.0f;
    v4f acc = {0.f, 0.f, 0.f, 0.f};
    if (M != -INFINITY) {
#pragma unroll
        for (int s = 0; s < S; ++s) {
            const float a = exp2f(m[s] - M);  // a part with no valid key has m = -inf: weight 0
            L += a * l[s];
            Llse += a * ll[s];
            acc += a * o[s];
        }
    }
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    const int64_t oo = ((int64_t)row * Hm + h) * 512 + 4 * t;
    if constexpr (ROPE) {
        // channels 4t .. 4t+3 are two RoPE pairs: turned back from 448 on, then cast
        float f[4] = {acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
        if (4 * t >= 448) {
            const float* c = rope_cs + (int64_t)row * 64 + (4 * t - 448);
            rope_pair(f[0], f[1], c[0], c[1], -1.0f);
            rope_pair(f[2], f[3], c[2], c[3], -1.0f);
        }
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + oo) =
            uint2{bf16_rne(f[0]) | (bf16_rne(f[1]) << 16), bf16_rne(f[2]) | (bf16_rne(f[3]) << 16)};
    } else {
        *reinterpret_cast<v4f*>(reinterpret_cast<float*>(out) + oo) = acc * inv;
    }
    if (lse && t == 0) lse[(int64_t)row * Hm + h] = Llse > 0.0f ? (M + log2f(Llse)) * 0.69314718055994531f : -INFINITY;
}

}  // namespace

hipError_t launch_gather_dequant(const csa2_batch* b, Geometry g, int kv_fmt, const uint8_t* kv, const uint8_t* kv_sc,
                                 const int32_t* idx, int K, uint16_t* out, hipStream_t s) {
    if (kv_fmt == kKvE4)
        hipLaunchKernelGGL(k_gather_dequant<kKvE4>, dim3(K, g.total_q), dim3(64), 0, s, kv, kv_sc, b->d_entry_off,
                           b->d_row_seq, idx, K, out);
    else
        hipLaunchKernelGGL(k_gather_dequant<kKvMx>, dim3(K, g.total_q), dim3(64), 0, s, kv, kv_sc, b->d_entry_off,
                           b->d_row_seq, idx, K, out);
    return hipGetLastError();
}

int attn_splits(const Geometry& g, int Hm, int K, int W) {
    if (attn_rows_ok(g, Hm)) return 1;
    // split the key blocks of a (row, head group) over several workgroups when
    // the grid would otherwise leave CUs idle
    const int units = g.total_q * (Hm / HG);
    const int max_blocks = (K + W + KB - 1) / KB;
    int S = (kAttnTargetWgs + units - 1) / units;
    S = S < 1 ? 1 : (S > kMaxSplit ? kMaxSplit : S);
    return S < max_blocks ? S : max_blocks;
}

size_t attn_ws_bytes(const Geometry& g, int Hm, int S) {
    return S <= 1 ? 0 : (size_t)g.total_q * (Hm / HG) * S * (HG * 516) * sizeof(float);
}

hipError_t launch_sparse_attn(const AttnLaunch& a, hipStream_t s) {
    const bool swa8 = a.sw->fmt == CSA2_SWA_MXFP8;
    if (attn_rows_ok(a.g, a.Hm)) return launch_sparse_attn_rows(a, s);
    const int n_hg = a.Hm / HG;
    int S = attn_splits(a.g, a.Hm, a.K, a.sw->window);
    while (S > 1 && attn_ws_bytes(a.g, a.Hm, S) > a.ws_bytes) --S;  // use what the workspace allows
    const int rows8 = (a.g.total_q + 7) / 8 * 8;
    const unsigned nblk = (unsigned)rows8 * (unsigned)n_hg * (unsigned)S;
    float* part = S > 1 ? (float*)a.ws : nullptr;
    // two pipes per workgroup only where the grid leaves most CUs idle (latency
    // is all that counts there); otherwise one pipe, two workgroups per CU
    const bool rope = a.rope_cs != nullptr;
    const uint16_t* qv = a.q;
    void* ov = rope ? (void*)a.out16 : (void*)a.out;
#define CSA2_ATTN(NP, KF, SF, RP)                                                                                  \
    hipLaunchKernelGGL((k_sparse_attn<NP, KF, SF, RP>), dim3(nblk), dim3(256 * NP), 0, s, qv, a.Hm, a.kv, a.kv_sc, a.idx, \
                       a.K, a.swa, a.sw->d_row_off, a.sw->d_pos0, a.sw->d_replay_s, a.sw->window, a.b->d_entry_off, \
                       a.b->d_row_seq, a.b->d_q_pos, a.scale * 1.4426950408889634f, ov, a.lse, a.g.total_q,     \
                       n_hg, S, part, a.rope_cs)
#define CSA2_ATTN_RP(NP, KF, SF)                        \
    do {                                                \
        if (rope) CSA2_ATTN(NP, KF, SF, 1);             \
        else CSA2_ATTN(NP, KF, SF, 0);                  \
    } while (0)
#define CSA2_ATTN_NP(KF, SF)                  \
    do {                                      \
        if (nblk <= kAttnTwoPipeWgs)          \
            CSA2_ATTN_RP(2, KF, SF);          \
        else                                  \
            CSA2_ATTN_RP(1, KF, SF);          \
    } while (0)
    if (a.kv_fmt == kKvE4) {
        if (swa8) CSA2_ATTN_NP(kKvE4, kSwaMx8); else CSA2_ATTN_NP(kKvE4, kSwaBf16);
    } else {
        if (swa8) CSA2_ATTN_NP(kKvMx, kSwaMx8); else CSA2_ATTN_NP(kKvMx, kSwaBf16);
    }
#undef CSA2_ATTN_NP
#undef CSA2_ATTN_RP
#undef CSA2_ATTN
    if (S > 1) {
        const dim3 cg((unsigned)(a.g.total_q * a.Hm));
        switch (S) {
#define CSA2_COMBINE(N)                                                                                           \
    case N:                                                                                                       \
        if (rope)                                                                                                 \
            hipLaunchKernelGGL((k_attn_combine<N, 1>), cg, dim3(128), 0, s, part, a.Hm, n_hg, ov, a.lse, a.rope_cs); \
        else                                                                                                      \
            hipLaunchKernelGGL((k_attn_combine<N, 0>), cg, dim3(128), 0, s, part, a.Hm, n_hg, ov, a.lse, a.rope_cs); \
        break;
            CSA2_COMBINE(2) CSA2_COMBINE(3) CSA2_COMBINE(4) CSA2_COMBINE(5)
            CSA2_COMBINE(6) CSA2_COMBINE(7) CSA2_COMBINE(8)
#undef CSA2_COMBINE
            default: return hipErrorInvalidValue;
        }
    }
    return hipGetLastError();
}

}  // namespace csa2
