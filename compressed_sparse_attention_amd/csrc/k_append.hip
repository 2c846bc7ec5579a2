// Cache append: a new main-KV entry is rotated and quantised into its row.
//
// Report "DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache Compression",
// section 2.4.4: the main KV is quantised after RoPE, all 512 channels,
// rotated part included, in E2M1 with one E4M3 scale per 16 channels (NVFP4's
// layout without its second-level scale); the OCP MXFP4 form (one E8M0 per 32
// channels) is this library's other main-KV format.  Section 4.2.1: the RoPE
// part of the 512-channel latent is 64 dimensions.
//
// Readings: the rotated channels are 448..511, pair i = (448 + 2i, 449 + 2i)
// turned by the caller's (cos, sin) of that pair, each output one rounded
// product difference or sum (no fused multiply-add).  The quantiser decides
// in fp32 on correctly rounded quotients: E4M3/16: X = E4M3(amax / 6) to
// nearest even (2^-9 where that is 0); MXFP4/32: X = 2^(floor(log2 amax) - 2)
// clamped to the E8M0 range (2^0 for an all-zero block); codes E2M1(x / X) to
// nearest even, saturating at 6.
//
// One wave per entry: lane l holds channels 8l .. 8l + 7, so a 16-channel
// block is a lane pair and a 32-channel block a lane quad; the 256-byte code
// row is one dword per lane.
#include <hip/hip_runtime.h>

#include "csa2_internal.h"

namespace csa2 {
namespace {

// nearest E2M1 code of q (ties to the even code), saturating at 6
__device__ __forceinline__ uint32_t e2m1_code_rne(float q) {
    const float a = fabsf(q);
    uint32_t c = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) + (a >= 3.5f) + (a > 5.0f);
    return c | (q < 0.0f ? 8u : 0u);
}

// nearest E4M3 code of q >= 0 (ties to even), saturating at 448 (code 126)
__device__ __forceinline__ uint32_t e4m3_code_rne(float q) {
    if (!(q < 448.0f)) return 126u;
    if (q < 0.015625f) return (uint32_t)rintf(q * 512.0f);  // subnormal steps of 2^-9 (8 -> 2^-6, code 8)
    int e;
    const float m = frexpf(q, &e);                           // q = m 2^e, m in [0.5, 1)
    const uint32_t m3 = (uint32_t)rintf((m * 2.0f - 1.0f) * 8.0f);  // exact scalings, then one rounding
    const uint32_t c = ((uint32_t)(e - 1 + 7) << 3) + m3;   // m3 = 8 carries into the exponent
    return c < 126u ? c : 126u;
}

__device__ __forceinline__ float e4m3_value(uint32_t c) {
    const uint32_t e = c >> 3, m = c & 7u;
    return e == 0 ? ldexpf((float)m, -9) : ldexpf((float)(8 + m), (int)e - 10);
}

template <int KVF>
__global__ __launch_bounds__(256) void k_kv_append(const float* __restrict__ x, const float* __restrict__ cs,
                                                   const int64_t* __restrict__ dst, int64_t n, int64_t rows,
                                                   uint8_t* __restrict__ kv, uint8_t* __restrict__ kv_sc) {
    const int64_t e = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (e >= n) return;
    const int64_t r = dst[e];
    if (r < 0 || r >= rows) return;  // rows outside the cache are left alone (the host cannot check them)

    float v[8];
    {
        const float4* src = reinterpret_cast<const float4*>(x + e * 512 + 8 * lane);
        const float4 a = src[0], b = src[1];
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
    if (lane >= 56) {  // channels 448 .. 511: pairs 4 (lane - 56) .. + 3
        // each product rounded on its own: the default contraction would fuse
        // a cos - b sin into one multiply-add, which rounds differently
#pragma clang fp contract(off)
        const float4* cp = reinterpret_cast<const float4*>(cs + (e * 32 + 4 * (lane - 56)) * 2);
        const float4 c0 = cp[0], c1 = cp[1];
        const float co[4] = {c0.x, c0.z, c1.x, c1.z}, si[4] = {c0.y, c0.w, c1.y, c1.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float a = v[2 * k], b = v[2 * k + 1];
            v[2 * k] = a * co[k] - b * si[k];
            v[2 * k + 1] = a * si[k] + b * co[k];
        }
    }

    float am = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(v[i]));
    am = fmaxf(am, __shfl_xor(am, 1));
    if constexpr (KVF == 0) am = fmaxf(am, __shfl_xor(am, 2));

    uint32_t sc;
    float X = 1.0f;
    int se = 0;
    if constexpr (KVF == 1) {
        sc = e4m3_code_rne(__fdiv_rn(am, 6.0f));
        sc = sc ? sc : 1u;
        X = e4m3_value(sc);
    } else {
        if (am > 0.0f) {
            int ex;
            frexpf(am, &ex);  // am = m 2^ex, m in [0.5, 1): floor(log2 am) = ex - 1
            se = ex - 3 < -127 ? -127 : ex - 3;
        }
        sc = (uint32_t)(se + 127);
    }
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float q = KVF == 1 ? __fdiv_rn(v[i], X) : ldexpf(v[i], -se);  // a power of two scales exactly
        word |= e2m1_code_rne(q) << (4 * i);
    }
    *reinterpret_cast<uint32_t*>(kv + r * 256 + 4 * lane) = word;
    if constexpr (KVF == 1) {
        if ((lane & 1) == 0) kv_sc[r * 32 + (lane >> 1)] = (uint8_t)sc;
    } else {
        if ((lane & 3) == 0) kv_sc[r * 16 + (lane >> 2)] = (uint8_t)sc;
    }
}

// Compressor (reading note "DeepSeek V4.1 Flash: Pushing the Limits of KV
// Cache Compression": C = H W^KV are the KV rows and Z = H W^Z their
// compression weights; CSA2 drops V4's overlapping windows and absolute
// position embedding).  Reading: entry j combines tokens jm .. jm + m - 1 per
// channel with the softmax over those tokens of Z.  A thread owns 4 channels
// of one entry (128 threads an entry, 2 entries a workgroup).
__global__ __launch_bounds__(256) void k_compress(const float* __restrict__ c_tok, const float* __restrict__ z_tok,
                                                  int64_t n, int m, float* __restrict__ out) {
    const int64_t j = (int64_t)blockIdx.x * 2 + (threadIdx.x >> 7);
    if (j >= n) return;
    const int c0 = 4 * (threadIdx.x & 127);
    const int64_t t0 = j * m;
    float mx[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    for (int i = 0; i < m; ++i) {
        const float4 z = *reinterpret_cast<const float4*>(z_tok + (t0 + i) * 512 + c0);
        mx[0] = fmaxf(mx[0], z.x); mx[1] = fmaxf(mx[1], z.y); mx[2] = fmaxf(mx[2], z.z); mx[3] = fmaxf(mx[3], z.w);
    }
    float num[4] = {0.f, 0.f, 0.f, 0.f}, den[4] = {0.f, 0.f, 0.f, 0.f};
    for (int i = 0; i < m; ++i) {
        const float4 z = *reinterpret_cast<const float4*>(z_tok + (t0 + i) * 512 + c0);
        const float4 c = *reinterpret_cast<const float4*>(c_tok + (t0 + i) * 512 + c0);
        const float zz[4] = {z.x, z.y, z.z, z.w}, cc[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float w = expf(zz[k] - mx[k]);  // <= 1: the token with the largest weight gives 1
            num[k] += w * cc[k];
            den[k] += w;
        }
    }
    *reinterpret_cast<float4*>(out + j * 512 + c0) =
        float4{num[0] / den[0], num[1] / den[1], num[2] / den[2], num[3] / den[3]};
}

// Indexer-K projection (reading note "DeepSeek V4.1 Flash: Pushing the Limits
// of KV Cache Compression", configuration section: indexer K is projected
// directly from the main KV; the report, section 2.4.4: indexer keys in
// MXFP4).  y = x W over the entry's 512 channels (after RoPE: with the
// entry's angles cs, x is the entry before RoPE and its channels 448..511 are
// turned on the way into LDS exactly as the append turns them), each output the fp32
// multiply-add chain in ascending channel order (the order the results are
// defined in), then E2M1 codes with the OCP MX scale 2^(floor(log2 amax) - 2)
// per row (KF 0) or per 32 channels (KF 1).  64 entries a workgroup; thread t
// owns outputs 8 (t % 16) .. + 7 of entries 4 (t / 16) .. + 3, so the 16
// threads of an entry quad are one 16-lane group.  Per 64-channel step the
// entries' channels (transposed: one 16-byte read gives a channel of 4
// entries) and that slice of W are staged in LDS: three 16-byte reads feed 32
// multiply-adds.
template <int KF>
__global__ __launch_bounds__(256) void k_index_k_project(const float* __restrict__ x, const float* __restrict__ cs,
                                                         const float* __restrict__ W, const int64_t* __restrict__ dst,
                                                         int64_t n, int64_t rows, uint8_t* __restrict__ k_fp4,
                                                         uint8_t* __restrict__ k_sc) {
    __shared__ __attribute__((aligned(16))) float xs[64][64 + 4];  // [channel][entry], padded rows
    __shared__ __attribute__((aligned(16))) float ws[64][128];
    const int t = threadIdx.x;
    const int64_t e0 = (int64_t)blockIdx.x * 64;
    const int eq = t >> 4, og = t & 15;
    float acc[4][8];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[j][i] = 0.0f;
    for (int kt = 0; kt < 8; ++kt) {
        __syncthreads();  // the previous step's tiles are consumed
        // 64 entries x 16 float4 of this step's channels: thread t takes float4
        // c4 = t % 16 of entries t / 16 + 16 u.  Entries past n re-read entry
        // n - 1 (their outputs are not stored), so that every load is
        // unconditional and all are issued before the first is used.
        const int c4 = t & 15;
        float4 v[4];
        int64_t e[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t eu = e0 + (t >> 4) + 16 * u;
            e[u] = eu < n ? eu : n - 1;
            v[u] = reinterpret_cast<const float4*>(x + e[u] * 512 + 64 * kt)[c4];
        }
        if (kt == 7 && cs != nullptr) {
            // channels 448 + 4 c4 .. + 3 are pairs 2 c4 and 2 c4 + 1, turned as
            // the append turns them: rounded products, then one rounded
            // difference or sum (no fused multiply-add)
#pragma clang fp contract(off)
            float4 a[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) a[u] = reinterpret_cast<const float4*>(cs + e[u] * 64)[c4];  // cos, sin, cos, sin
#pragma unroll
            for (int u = 0; u < 4; ++u)
                v[u] = float4{v[u].x * a[u].x - v[u].y * a[u].y, v[u].x * a[u].y + v[u].y * a[u].x,
                              v[u].z * a[u].z - v[u].w * a[u].w, v[u].z * a[u].w + v[u].w * a[u].z};
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int el = (t >> 4) + 16 * u;
            xs[4 * c4 + 0][el] = v[u].x;
            xs[4 * c4 + 1][el] = v[u].y;
            xs[4 * c4 + 2][el] = v[u].z;
            xs[4 * c4 + 3][el] = v[u].w;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {  // 64 rows of W, 32 float4 each
            const int i = t + 256 * u, kr = i >> 5, c4 = i & 31;
            reinterpret_cast<float4*>(&ws[kr][0])[c4] = reinterpret_cast<const float4*>(W + (int64_t)(64 * kt + kr) * 128)[c4];
        }
        __syncthreads();
#pragma unroll 2
        for (int k = 0; k < 64; ++k) {
            const float4 xv = *reinterpret_cast<const float4*>(&xs[k][4 * eq]);
            const float4 w0 = reinterpret_cast<const float4*>(&ws[k][8 * og])[0];
            const float4 w1 = reinterpret_cast<const float4*>(&ws[k][8 * og])[1];
            const float xe[4] = {xv.x, xv.y, xv.z, xv.w};
            const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[j][i] = __builtin_fmaf(xe[j], wv[i], acc[j][i]);
        }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        // block maxima over the entry's 16 threads (KF 0) or over 4 (KF 1)
        float am = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(acc[j][i]));
        am = fmaxf(am, __shfl_xor(am, 1));
        am = fmaxf(am, __shfl_xor(am, 2));
        if constexpr (KF == 0) {
            am = fmaxf(am, __shfl_xor(am, 4));
            am = fmaxf(am, __shfl_xor(am, 8));
        }
        int se = 0;
        if (am > 0.0f) {
            int ex;
            frexpf(am, &ex);
            se = ex - 3 < -127 ? -127 : ex - 3;
        }
        uint32_t word = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) word |= e2m1_code_rne(ldexpf(acc[j][i], -se)) << (4 * i);
        const int64_t e = e0 + 4 * eq + j;
        if (e >= n) continue;
        const int64_t r = dst[e];
        if (r < 0 || r >= rows) continue;
        *reinterpret_cast<uint32_t*>(k_fp4 + r * 64 + 4 * og) = word;
        if constexpr (KF == 1) {
            if ((og & 3) == 0) k_sc[r * 4 + (og >> 2)] = (uint8_t)(se + 127);
        } else {
            if (og == 0) k_sc[r] = (uint8_t)(se + 127);
        }
    }
}

// RoPE and cast around attention (the report's kernel flow: a fused
// "RoPE-attention-RoPE-cast" kernel rotates the query before attention and
// turns the output's rotated part back after it, then casts).  The pairs and
// angles are the append's (channels 448..511, caller-given cos/sin per row);
// `inverse` negates the angle.  64 threads a head row, 8 channels a thread.
__global__ __launch_bounds__(256) void k_rope_cast(const float* __restrict__ in, const float* __restrict__ cs,
                                                   int64_t n_rows, int heads, int inverse, uint16_t* __restrict__ out) {
    const int64_t hr = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // head row = row * heads + head
    if (hr >= n_rows * heads) return;
    const int lane = threadIdx.x & 63;
    const int64_t r = hr / heads;
    float v[8];
    {
        const float4* src = reinterpret_cast<const float4*>(in + hr * 512 + 8 * lane);
        const float4 a = src[0], b = src[1];
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
    if (lane >= 56) {
        // each product rounded on its own, as in the append
#pragma clang fp contract(off)
        const float4* cp = reinterpret_cast<const float4*>(cs + (r * 32 + 4 * (lane - 56)) * 2);
        const float4 c0 = cp[0], c1 = cp[1];
        const float co[4] = {c0.x, c0.z, c1.x, c1.z};
        const float sg = inverse ? -1.0f : 1.0f;  // exact negation
        const float si[4] = {sg * c0.y, sg * c0.w, sg * c1.y, sg * c1.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float a = v[2 * k], b = v[2 * k + 1];
            v[2 * k] = a * co[k] - b * si[k];
            v[2 * k + 1] = a * si[k] + b * co[k];
        }
    }
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) w[k] = bf16_rne(v[2 * k]) | (bf16_rne(v[2 * k + 1]) << 16);
    *reinterpret_cast<uint4*>(out + hr * 512 + 8 * lane) = uint4{w[0], w[1], w[2], w[3]};
}

}  // namespace

hipError_t launch_rope_cast(int64_t n_rows, int heads, const float* in, const float* cs, int inverse, uint16_t* out,
                            hipStream_t s) {
    const int64_t hrows = n_rows * heads;
    hipLaunchKernelGGL(k_rope_cast, dim3((unsigned)((hrows + 3) / 4)), dim3(256), 0, s, in, cs, n_rows, heads, inverse,
                       out);
    return hipGetLastError();
}

hipError_t launch_index_k_project(int64_t n, const float* x, const float* cs, const float* W, const int64_t* dst,
                                  int64_t rows, int mx, uint8_t* k_fp4, uint8_t* k_sc, hipStream_t s) {
    const dim3 grid((unsigned)((n + 63) / 64));
    if (mx)
        hipLaunchKernelGGL(k_index_k_project<1>, grid, dim3(256), 0, s, x, cs, W, dst, n, rows, k_fp4, k_sc);
    else
        hipLaunchKernelGGL(k_index_k_project<0>, grid, dim3(256), 0, s, x, cs, W, dst, n, rows, k_fp4, k_sc);
    return hipGetLastError();
}

hipError_t launch_compress(int64_t n, int m, const float* c_tok, const float* z_tok, float* out, hipStream_t s) {
    hipLaunchKernelGGL(k_compress, dim3((unsigned)((n + 1) / 2)), dim3(256), 0, s, c_tok, z_tok, n, m, out);
    return hipGetLastError();
}

hipError_t launch_kv_append(int64_t n, const float* x, const float* cs, const int64_t* dst, int64_t rows, int kv_fmt,
                            uint8_t* kv, uint8_t* kv_sc, hipStream_t s) {
    const dim3 grid((unsigned)((n + 3) / 4));
    if (kv_fmt == 1)
        hipLaunchKernelGGL(k_kv_append<1>, grid, dim3(256), 0, s, x, cs, dst, n, rows, kv, kv_sc);
    else
        hipLaunchKernelGGL(k_kv_append<0>, grid, dim3(256), 0, s, x, cs, dst, n, rows, kv, kv_sc);
    return hipGetLastError();
}

}  // namespace csa2
