// Sparse latent attention for many query rows (prefill chunks, replays): one
// workgroup per (query row, 64 heads), so a row's selected entries and window
// rows are dequantised once for all of its heads (the split kernel in
// k_attn.hip stages them once per 16-head group).
//
// Report "DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache Compression":
// section 2.3 (each query attends to its Top-K entries together with the
// layer-local sliding-window KV), section 2.4.4 (FP4 main KV dequantised before
// attention), section 4.2.1 (64 query heads of dim 512 sharing one latent).
// Course notes "3. 通用基础设施", section 3.2.2: query i sees SWA keys
// [max(s, i-W+1), i].
//
// 4 waves; wave w owns heads 16w .. 16w+15 of the group for the whole row, so
// the softmax needs no exchange between waves.  Per block of 64 keys (the SWA
// rows first, then the selected entries):
//   stage  the block into LDS as bf16 rows (each thread one key, 128 channels);
//   S^T    = K Q^T on v_mfma_f32_16x16x32_bf16, four 16-key tiles: A = key rows
//          from LDS, B = the wave's 16 query rows held in registers.  Lane l
//          receives head l%16 and keys 16t + 4(l/16) + i of tile t, i.e. every
//          head's scores sit in the four lanes l%16 + 16g;
//   softmax online per head in fp32 (base 2); the weights of keys
//          32s + 16(e/4) + 4g + e%4, e = 0..7, form the A operand of P V step
//          s in the lane that computed them, as a bf16 pair (hi + lo);
//   P V    on the same MFMA: B = V read transposed from LDS
//          (ds_read_b64_tr_b16) in the same key order, O = 16 heads x 512
//          channels in registers.
// The waves share data through LDS only, so their barriers order LDS only.
// Two workgroups share a CU (75 KB of LDS each), so one stages while the
// other computes.  Used only where the grid fills the chip without splitting
// a row's keys: with splits every part writes a 64-head partial (128 KB), and
// at 64 rows the parts and their merge took 38 us against 33 us for the
// 16-head kernel.  Measured alternatives: one workgroup per CU with a
// double-buffered block, the next block's loads in flight during the
// products and the accumulators in AGPRs (one wave per SIMD) ran slower
// (1.77 against 1.38 ms per prefill_c3 layer); explicit two-stage operand
// buffers at two workgroups per CU spill.
#include "attn_common.h"

namespace csa2 {
namespace {

using namespace attn;

template <int KVF, int SWF, int ROPE>
__global__ __launch_bounds__(256, 2) void k_sparse_attn_rows(
    const uint16_t* __restrict__ q, int Hm, const uint8_t* __restrict__ kv, const uint8_t* __restrict__ kv_sc,
    const int32_t* __restrict__ idx, int K, const void* __restrict__ swa, const int64_t* __restrict__ swa_row_off,
    const int32_t* __restrict__ swa_pos0, const int32_t* __restrict__ replay_s, int W,
    const int64_t* __restrict__ entry_off, const int32_t* __restrict__ row_seq, const int32_t* __restrict__ q_pos,
    float scale_log2, void* __restrict__ out, float* __restrict__ lse, int total_q, int n_hg,
    const float* __restrict__ rope_cs) {
    __shared__ __attribute__((aligned(16))) uint16_t kl[KB * LROW];
    __shared__ __attribute__((aligned(16))) int kvalid[KB];  // read as int4
    __shared__ int32_t kidx[kMaxK];
    __shared__ int nsel_sh;

    const int row = blockIdx.x / n_hg, hg = blockIdx.x % n_hg;
    if (row >= total_q) return;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lg = lane >> 4, li = lane & 15;

    // ---- prologue: the index row, then the wave's query rows
    const int32_t* irow = idx + (int64_t)row * K;
    int32_t ir[kMaxK / 256];
#pragma unroll
    for (int i = 0; i < kMaxK / 256; ++i) {
        const int s = tid + 256 * i;
        ir[i] = s < K ? irow[s] : -1;
    }
    __builtin_amdgcn_sched_barrier(0);
    const int h0 = 64 * hg + 16 * wave;  // the wave's first head
    v8bf Q[16];
    const float* row_cs = ROPE ? rope_cs + (int64_t)row * 64 : nullptr;
    {
        const int64_t qr = ((int64_t)row * Hm + h0 + li) * 512 + 8 * lg;
        load_q16<ROPE>(Q, q, qr, lg, row_cs);
    }
    asm volatile("" ::: "memory");

    const int b = row_seq[row];
    const int64_t t = q_pos[row];
    const int64_t e0 = entry_off[b];
    const int64_t n_ent = entry_off[b + 1] - e0;
    const int64_t s_rep = replay_s ? (int64_t)replay_s[b] : 0;
    int64_t u_lo = t - W + 1;
    u_lo = u_lo > s_rep ? u_lo : s_rep;
    const int n_swa = t >= u_lo ? (int)(t - u_lo + 1) : 0;
    const int64_t swa_r0 = swa_row_off[b] + (u_lo - swa_pos0[b]);

    if (tid == 0) nsel_sh = 0;
    lds_barrier();
    {
        int last = 0;
#pragma unroll
        for (int i = 0; i < kMaxK / 256; ++i) {
            const int s = tid + 256 * i;
            if (s < K) {
                const int32_t j = (ir[i] >= 0 && ir[i] < n_ent) ? ir[i] : -1;  // out-of-range entries read as empty
                kidx[s] = j;
                if (j >= 0) last = s + 1;
            }
        }
        if (last) atomicMax(&nsel_sh, last);
    }
    lds_barrier();
    const int n_keys = n_swa + nsel_sh;
    const int n_blk = (n_keys + KB - 1) / KB;


    // this thread stages key `skey` of a block, channels 128 part .. +128;
    // 16 consecutive lanes take 16 keys of one part (distinct LDS banks)
    constexpr int CP = 128;
    constexpr int NB = CP / 32;
    const int skey = (tid & 15) + 16 * (tid >> 6), part = (tid >> 4) & 3;
    uint16_t* const kdst = kl + skey * LROW + CP * part;
    auto stage = [&](int blk) {
        const int vk = KB * blk + skey;
        int valid = 0;
        if (vk < n_swa) {
            valid = 1;
            if constexpr (SWF == kSwaMx8) {
                const uint8_t* rb = reinterpret_cast<const uint8_t*>(swa) + (swa_r0 + vk) * 528;
                v4i sw[CP / 16];
#pragma unroll
                for (int i = 0; i < CP / 16; ++i) sw[i] = ld16(rb + CP * part + 16 * i);
                const uint32_t swsc = *reinterpret_cast<const uint32_t*>(rb + 512 + 4 * part);
#pragma unroll
                for (int i = 0; i < NB; ++i) {
                    const float sc = e8m0_f32((swsc >> (8 * i)) & 255u);
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        const uint32_t w0 = (uint32_t)sw[2 * i + d / 2][2 * (d % 2)];
                        const uint32_t w1 = (uint32_t)sw[2 * i + d / 2][2 * (d % 2) + 1];
                        auto a0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, sc, false);
                        auto a1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, sc, true);
                        auto b0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, sc, false);
                        auto b1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, sc, true);
                        *reinterpret_cast<v8bf*>(kdst + 32 * i + 8 * d) =
                            v8bf{a0[0], a0[1], a1[0], a1[1], b0[0], b0[1], b1[0], b1[1]};
                    }
                }
            } else {
                const uint16_t* src = reinterpret_cast<const uint16_t*>(swa) + (swa_r0 + vk) * 512 + CP * part;
#pragma unroll
                for (int h = 0; h < 2; ++h) {  // two halves of 8 loads (register budget)
                    v4i sw[CP / 16];
#pragma unroll
                    for (int i = 0; i < CP / 16; ++i) sw[i] = ld16(src + 64 * h + 8 * i);
#pragma unroll
                    for (int i = 0; i < CP / 16; ++i) *reinterpret_cast<v4i*>(kdst + 64 * h + 8 * i) = sw[i];
                }
            }
        } else if (vk < n_keys) {
            const int32_t j = kidx[vk - n_swa];
            if (j >= 0) {
                valid = 1;
                const int64_t e = e0 + j;
                const uint8_t* src = kv + e * 256 + (CP / 2) * part;
                v4i pc[NB];
#pragma unroll
                for (int i = 0; i < NB; ++i) pc[i] = ld16(src + 16 * i);
                if constexpr (KVF == kKvE4) {
                    const uint2 w2 = *reinterpret_cast<const uint2*>(kv_sc + e * 32 + 8 * part);
#pragma unroll
                    for (int i = 0; i < NB; ++i) {
                        const uint32_t w = i < 2 ? w2.x : w2.y;
                        const float s0 = e4m3_f32((w >> (16 * (i & 1))) & 255u);
                        const float s1 = e4m3_f32((w >> (16 * (i & 1) + 8)) & 255u);
#pragma unroll
                        for (int d = 0; d < 4; ++d)
                            *reinterpret_cast<v4i*>(kdst + 32 * i + 8 * d) =
                                fp4x8_to_bf16_mul((uint32_t)pc[i][d], d < 2 ? s0 : s1);
                    }
                } else {
                    const uint32_t psc = *reinterpret_cast<const uint32_t*>(kv_sc + e * 16 + 4 * part);
#pragma unroll
                    for (int i = 0; i < NB; ++i) {
                        const float sc = e8m0_f32((psc >> (8 * i)) & 255u);
#pragma unroll
                        for (int d = 0; d < 4; ++d)
                            *reinterpret_cast<v4i*>(kdst + 32 * i + 8 * d) = fp4x8_to_bf16((uint32_t)pc[i][d], sc);
                    }
                }
            }
        }
        if (!valid) {
#pragma unroll
            for (int i = 0; i < CP / 8; ++i) *reinterpret_cast<v4i*>(kdst + 8 * i) = v4i{0, 0, 0, 0};
        }
        if (part == 0) kvalid[skey] = valid;
    };

    v4f O[32];
#pragma unroll
    for (int nt = 0; nt < 32; ++nt) O[nt] = v4f{0.f, 0.f, 0.f, 0.f};
    // running max and sum of head h0 + li (the same in the four lanes of a head)
    float m_run = -INFINITY, l_run = 0.0f;

    for (int blk = 0; blk < n_blk; ++blk) {
        if (blk > 0) lds_barrier();  // every wave is done with the previous block
        stage(blk);
        lds_barrier();

        // S^T = K Q^T: four independent accumulation chains (key tiles)
        v4f S[4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int ks = 0; ks < 16; ++ks) {
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                const v8bf Ak = __builtin_bit_cast(v8bf, *reinterpret_cast<const v4i*>(kl + (16 * tt + li) * LROW + 32 * ks + 8 * lg));
                S[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Ak, Q[ks], S[tt], 0, 0, 0);
            }
        }
        // scaled logits; keys that are not there score -inf
        float p[16];
        float mx = -INFINITY;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            const int4 ok = *reinterpret_cast<const int4*>(kvalid + 16 * tt + 4 * lg);
            const int okv[4] = {ok.x, ok.y, ok.z, ok.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                p[4 * tt + i] = okv[i] ? S[tt][i] * scale_log2 : -INFINITY;
                mx = fmaxf(mx, p[4 * tt + i]);
            }
        }
        mx = xor_max<16>(mx);
        mx = xor_max<32>(mx);
        const float m_new = fmaxf(m_run, mx);
        float alpha;
        if (m_new == -INFINITY) {  // nothing valid yet
            alpha = 1.0f;
#pragma unroll
            for (int i = 0; i < 16; ++i) p[i] = 0.0f;
        } else {
            // arguments are <= 0 (or -inf): the hardware exp2
            alpha = __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
            for (int i = 0; i < 16; ++i) p[i] = __builtin_amdgcn_exp2f(p[i] - m_new);
        }
        // P V operands: step s2 takes tiles 2 s2 and 2 s2 + 1, element e = key
        // 32 s2 + 16 (e / 4) + 4 lg + e % 4; each weight as a bf16 pair (hi + lo)
        // The sum normalises with the fp32 weights: a pair holds a weight to
        // about 2^-16 of it, far inside the output tolerance.
        v8bf P[2], Plo[2];
        float r4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float pv = p[4 * (2 * s2 + e / 4) + e % 4];
                const __bf16 pb = (__bf16)pv;
                P[s2][e] = pb;
                Plo[s2][e] = (__bf16)(pv - (float)pb);
                r4[e % 4] += pv;
            }
        float rs = (r4[0] + r4[1]) + (r4[2] + r4[3]);
        rs = xor_sum<16>(rs);
        rs = xor_sum<32>(rs);
        l_run = l_run * alpha + rs;
        m_run = m_new;
        // O rows are heads 4 lg + v: their alpha lives in lane 4 lg + v; the
        // rescale is skipped when no head's maximum moved
        if (__any(alpha != 1.0f)) {
            float av[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) av[v] = __shfl(alpha, 4 * lg + v);
#pragma unroll
            for (int nt = 0; nt < 32; ++nt)
#pragma unroll
                for (int v = 0; v < 4; ++v) O[nt][v] *= av[v];
        }
        // O += P V for channels 16 nt + li
#pragma unroll
        for (int nt = 0; nt < 32; ++nt) {
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                const uint16_t* a0 = kl + (32 * s2 + 4 * lg + (li >> 2)) * LROW + 16 * nt + 4 * (li & 3);
                const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(a0));
                const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(a0 + 16 * LROW));
                const v8s both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                const v8bf vb = __builtin_bit_cast(v8bf, both);
                O[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(P[s2], vb, O[nt], 0, 0, 0);
                O[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Plo[s2], vb, O[nt], 0, 0, 0);
            }
        }
    }

    // finalise: O / l for heads 4 lg + v
    const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;
    float iv[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) iv[v] = __shfl(inv, 4 * lg + v);
    // channel 16 nt + li is in the rotated part from nt = 28 on
    float2 ang[4] = {};
    if constexpr (ROPE) load_out_angles(ang, row_cs, li);
#pragma unroll
    for (int nt = 0; nt < 32; ++nt)
#pragma unroll
        for (int v = 0; v < 4; ++v)
            store_out<ROPE>(out, ((int64_t)row * Hm + h0 + 4 * lg + v) * 512 + 16 * nt + li, 16 * nt + li,
                            O[nt][v] * iv[v], nt >= 28, ang[nt >= 28 ? nt - 28 : 0]);
    if (lse && lg == 0)
        lse[(int64_t)row * Hm + h0 + li] = l_run > 0.0f ? (m_run + log2f(l_run)) * 0.69314718055994531f : -INFINITY;
}

}  // namespace

hipError_t launch_sparse_attn_rows(const AttnLaunch& a, hipStream_t s) {
    const int n_hg64 = a.Hm / 64;
    const dim3 grid((unsigned)(a.g.total_q * n_hg64));
    const bool swa8 = a.sw->fmt == CSA2_SWA_MXFP8;
    const bool rope = a.rope_cs != nullptr;
    const uint16_t* qv = a.q;
    void* ov = rope ? (void*)a.out16 : (void*)a.out;
#define CSA2_ROWS_RP(KF, SF, RP)                                                                                   \
    hipLaunchKernelGGL((k_sparse_attn_rows<KF, SF, RP>), grid, dim3(256), 0, s, qv, a.Hm, a.kv, a.kv_sc, a.idx, a.K, \
                       a.swa, a.sw->d_row_off, a.sw->d_pos0, a.sw->d_replay_s, a.sw->window, a.b->d_entry_off,     \
                       a.b->d_row_seq, a.b->d_q_pos, a.scale * 1.4426950408889634f, ov, a.lse, a.g.total_q, n_hg64, \
                       a.rope_cs)
#define CSA2_ROWS(KF, SF)                        \
    do {                                         \
        if (rope) CSA2_ROWS_RP(KF, SF, 1);       \
        else CSA2_ROWS_RP(KF, SF, 0);            \
    } while (0)
    if (a.kv_fmt == kKvE4) {
        if (swa8) CSA2_ROWS(kKvE4, kSwaMx8); else CSA2_ROWS(kKvE4, kSwaBf16);
    } else {
        if (swa8) CSA2_ROWS(kKvMx, kSwaMx8); else CSA2_ROWS(kKvMx, kSwaBf16);
    }
#undef CSA2_ROWS_RP
#undef CSA2_ROWS
    return hipGetLastError();
}

}  // namespace csa2
