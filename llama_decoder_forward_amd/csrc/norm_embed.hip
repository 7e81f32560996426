// Embedding gather and RMSNorm.
#include "common.h"

namespace {

constexpr int kThreads = 256;

// Row m of x = row tok of E (the reference's tok_embeddings lookup,
// walkthrough section 2).  Prefill at positions pos0..: m = b*T + t reads
// tok[b][pos0 + t]; decode (pos_dev != NULL, T == 1): row b reads
// tok[b][*pos_dev].
__global__ void embed_kernel(const char *E, const int32_t *tok, int64_t tok_ld, int T,
                             const int *pos_dev, int pos0, const int *pos_rows, const int2 *rowmap,
                             int64_t row_bytes, char *x)
{
    const int m = blockIdx.x;
    int b, col;
    locate_row(m, T, pos_dev, pos0, pos_rows, rowmap, b, col);
    int32_t id = tok[(int64_t)b * tok_ld + col];
    const uint4 *src = reinterpret_cast<const uint4 *>(E + (int64_t)id * row_bytes);
    uint4 *dst = reinterpret_cast<uint4 *>(x + (int64_t)m * row_bytes);
    for (int64_t i = threadIdx.x; i < row_bytes / 16; i += blockDim.x) dst[i] = src[i];
}

// Row i of out = row idx[i] of x (the last token of each varlen row).
__global__ void gather_rows_kernel(const char *x, const int *idx, int64_t row_bytes, char *out)
{
    const uint4 *src = reinterpret_cast<const uint4 *>(x + (int64_t)idx[blockIdx.x] * row_bytes);
    uint4 *dst = reinterpret_cast<uint4 *>(out + (int64_t)blockIdx.x * row_bytes);
    for (int64_t i = threadIdx.x; i < row_bytes / 16; i += blockDim.x) dst[i] = src[i];
}

__device__ __forceinline__ float block_sum(float v, float *red)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    if (l == 0) red[w] = v;
    __syncthreads();
    float t = 0.f;
    for (int i = 0; i < (int)(blockDim.x >> 6); i++) t += red[i];
    return t;
}

// RMSNorm (walkthrough section 3.2): r = 1/sqrt(mean(x^2) + eps) in fp32,
// y = round(round(x * r) * w).  One wave per row: 16-byte loads kept in
// registers (D <= 64 * 8 * RMS_VEC), a shuffle-only reduction, no barrier.
constexpr int RMS_VEC = 16;  // D up to 8192

__global__ __launch_bounds__(256) void rmsnorm_f16_kernel(const half_t *x, int64_t ldx, const half_t *w,
                                                          int M, int D, float eps, half_t *y, int y_lay)
{
#pragma clang fp contract(off)
    int blk = blockIdx.x;
    if (y_lay == ACT_TILED && (gridDim.x & 31) == 0) {
        // the four work-groups that write one 16-row group of the tile
        // layout (each 1 KiB block interleaves the 16 rows in 16-byte pieces)
        // run on one XCD (work-groups go to the eight XCDs round-robin), so
        // that the L2 they share merges the pieces into whole lines
        const int xcd = blk & 7, local = blk >> 3;
        blk = ((local >> 2) * 8 + xcd) * 4 + (local & 3);
    }
    const int row = blk * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (row >= M) return;
    const half8 *xr = reinterpret_cast<const half8 *>(x + (int64_t)row * ldx);
    half8 *yr = reinterpret_cast<half8 *>(y + (int64_t)row * D);
    const half8 *wr = reinterpret_cast<const half8 *>(w);
    const int nv = D / 8;
    half8 v[RMS_VEC], wv[RMS_VEC];
    // the weight row is loaded with x, so the two loads share one round trip
#pragma unroll
    for (int j = 0; j < RMS_VEC; j++) {
        const int i = lane + 64 * j;
        if (i < nv) {
            v[j] = xr[i];
            wv[j] = wr[i];
        }
    }
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < RMS_VEC; j++) {
        const int i = lane + 64 * j;
        if (i < nv) {
#pragma unroll
            for (int e = 0; e < 8; e++) { float f = (float)v[j][e]; ss += f * f; }
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
    const float r = __frcp_rn(__fsqrt_rn(ss / (float)D + eps));
#pragma unroll
    for (int j = 0; j < RMS_VEC; j++) {
        const int i = lane + 64 * j;
        if (i < nv) {
            half8 o;
#pragma unroll
            for (int e = 0; e < 8; e++) {
                half_t n = (half_t)((float)v[j][e] * r);
                o[e] = (half_t)((float)n * (float)wv[j][e]);
            }
            if (y_lay) *reinterpret_cast<half8 *>(y + act_offset(row, 8 * (int64_t)i, D, D, y_lay)) = o;
            else yr[i] = o;
        }
    }
}

// The same RMSNorm into the weight tile layout (ACT_TILED): one work-group of
// eight waves per half of a 16-row group, a wave per row with the arithmetic
// above.  A 1 KiB tile holds, for each of its four 8-column chunks, the 16
// rows' 16-byte pieces in row order, so rows 0..7 and rows 8..15 fill one
// 128-byte line each: the work-group stages half its rows' range at a time
// in LDS and writes whole lines.  The weight row is read once per
// work-group into LDS.  Rows past M (the last group) are written as zeros.
// D is a multiple of 512, so every lane holds J = D / 512 pieces and every
// bound below is uniform.
__global__ __launch_bounds__(512, 4) void rmsnorm_tiled_kernel(const half_t *x, int64_t ldx, const half_t *w, int M,
                                                               int D, float eps, half_t *y)
{
#pragma clang fp contract(off)
    extern __shared__ half8 sm[];  // weight row [D / 8], then [D / 64 tiles][4 chunks][8 rows]
    const int nv = D / 8, J = D / 512, KT = D / 32, half_kt = KT / 2;
    half8 *wl = sm, *st = sm + nv;
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int grp = blockIdx.x >> 1, sub = blockIdx.x & 1, row = grp * 16 + sub * 8 + wave;
    const half8 *wr = reinterpret_cast<const half8 *>(w);
    for (int i = tid; i < nv; i += 512) wl[i] = wr[i];
    const half8 *xr = reinterpret_cast<const half8 *>(x + (int64_t)row * ldx) + lane;
    half8 v[RMS_VEC];
    const bool live = row < M;  // uniform over the wave
#pragma unroll
    for (int j = 0; j < RMS_VEC; j++) v[j] = live && j < J ? xr[64 * j] : half8{};
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < RMS_VEC; j++) {
        if (j < J) {
#pragma unroll
            for (int e = 0; e < 8; e++) { float f = (float)v[j][e]; ss += f * f; }
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
    const float r = __frcp_rn(__fsqrt_rn(ss / (float)D + eps));
    __syncthreads();  // the weight row is in LDS
    half8 *yg = reinterpret_cast<half8 *>(y) + (int64_t)grp * KT * 64 + sub * 8;
    // piece i = lane + 64 j (elements 8i..8i+7) sits in k-tile 16 j + lane / 4,
    // chunk lane % 4.  Pass h stages the pieces of the odd or even j, i.e. the
    // k-tiles 16 j .. 16 j + 15 of those j (J is even), at staging tile
    // 16 (j / 2) + lane / 4.
#pragma unroll
    for (int h = 0; h < 2; h++) {
#pragma unroll
        for (int jj = 0; jj < RMS_VEC / 2; jj++) {
            const int j = 2 * jj + h;
            if (j < J) {
                const half8 wv = wl[lane + 64 * j];
                // the fp32 values of the row are converted again here rather
                // than kept from the sum of squares (that would hold twice
                // the registers)
                half8 vj = v[j];
                asm volatile("" : "+v"(vj));
                half8 o;
#pragma unroll
                for (int e = 0; e < 8; e++) {
                    half_t n = (half_t)((float)vj[e] * r);
                    o[e] = (half_t)((float)n * (float)wv[e]);
                }
                st[((jj * 16 + (lane >> 2)) * 4 + (lane & 3)) * 8 + wave] = o;
            }
        }
        __syncthreads();
        // q = (staging tile t, chunk, row): 8 rows of a chunk are one
        // 128-byte line at tile offset 256 chunk + 128 sub
        for (int q = tid; q < half_kt * 32; q += 512) {
            const int t = q >> 5, kt = ((t >> 4) * 2 + h) * 16 + (t & 15);
            yg[(int64_t)kt * 64 + ((q >> 3) & 3) * 16 + (q & 7)] = st[q];
        }
        __syncthreads();  // before the next pass reuses the staging area
    }
}

// The same RMSNorm for the few rows of a decode step: one row per work-group
// of eight waves, so the row's loads are spread over eight times as many
// CUs.  Thread t sums the squares of its elements 8t.., 8(t + 512).., ...,
// each wave adds by butterflies and the waves' sums are added in wave order:
// the order of the normalisation staged inside the one- and two-row
// products, so a row normalises to the same bits on either path.
// S > 0: x first receives the split-K partial sums part[S][M][D] of the
// residual product that wrote it (added in split order, then rounded as the
// residual epilogue rounds), and the new row is stored to xout (x itself).
// S is a template argument so that the loads of all S planes are issued
// before the first addition.
template <int S = 0>
__global__ __launch_bounds__(512) void rmsnorm_row_kernel(const half_t *x, int64_t ldx, const half_t *w, int D,
                                                          float eps, half_t *y, int y_lay, const float *part = nullptr,
                                                          half_t *xout = nullptr)
{
#pragma clang fp contract(off)
    constexpr bool PART = S > 0;
    __shared__ float pss[8];
    const int row = blockIdx.x, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const half8 *xr = reinterpret_cast<const half8 *>(x + (int64_t)row * ldx);
    const half8 *wr = reinterpret_cast<const half8 *>(w);
    const int nv = D / 8;
    constexpr int R = RMS_VEC / 8;  // D up to 8192
    half8 v[R], wv[R];
#pragma unroll
    for (int j = 0; j < R; j++) {
        const int i = tid + 512 * j;
        if (i < nv) {
            v[j] = xr[i];
            wv[j] = wr[i];
        }
    }
    if (PART) {
        const int64_t plane = (int64_t)gridDim.x * D;
#pragma unroll
        for (int j = 0; j < R; j++) {
            const int i = tid + 512 * j;
            if (i < nv) {
                const float4 *p = reinterpret_cast<const float4 *>(part + (int64_t)row * D + 8 * i);
                float4 b0[S > 0 ? S : 1], b1[S > 0 ? S : 1];
#pragma unroll
                for (int sp = 0; sp < S; sp++) {
                    b0[sp] = p[sp * plane / 4];
                    b1[sp] = p[sp * plane / 4 + 1];
                }
                float4 a0 = b0[0], a1 = b1[0];
#pragma unroll
                for (int sp = 1; sp < S; sp++) {
                    a0.x += b0[sp].x; a0.y += b0[sp].y; a0.z += b0[sp].z; a0.w += b0[sp].w;
                    a1.x += b1[sp].x; a1.y += b1[sp].y; a1.z += b1[sp].z; a1.w += b1[sp].w;
                }
                const float t[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
                for (int e = 0; e < 8; e++) v[j][e] = (half_t)((float)v[j][e] + (float)(half_t)t[e]);
                reinterpret_cast<half8 *>(xout + (int64_t)row * ldx)[i] = v[j];
            }
        }
    }
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < R; j++) {
        if (tid + 512 * j < nv) {
#pragma unroll
            for (int e = 0; e < 8; e++) { float f = (float)v[j][e]; ss += f * f; }
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
    if (lane == 0) pss[wave] = ss;
    __syncthreads();
    float t = 0.f;
#pragma unroll
    for (int ww = 0; ww < 8; ww++) t += pss[ww];
    const float r = __frcp_rn(__fsqrt_rn(t / (float)D + eps));
#pragma unroll
    for (int j = 0; j < R; j++) {
        const int i = tid + 512 * j;
        if (i < nv) {
            half8 o;
#pragma unroll
            for (int e = 0; e < 8; e++) {
                half_t n = (half_t)((float)v[j][e] * r);
                o[e] = (half_t)((float)n * (float)wv[j][e]);
            }
            if (y_lay) *reinterpret_cast<half8 *>(y + act_offset(row, 8 * (int64_t)i, D, D, y_lay)) = o;
            else reinterpret_cast<half8 *>(y + (int64_t)row * D)[i] = o;
        }
    }
}

__global__ void rmsnorm_f32_kernel(const float *x, int64_t ldx, const float *w, int D, float eps,
                                   float *y)
{
    __shared__ float red[kThreads / 64];
    const float *xr = x + (int64_t)blockIdx.x * ldx;
    float *yr = y + (int64_t)blockIdx.x * D;
    float ss = 0.f;
    for (int i = threadIdx.x; i < D; i += blockDim.x) ss += xr[i] * xr[i];
    float tot = block_sum(ss, red);
    float r = __frcp_rn(__fsqrt_rn(tot / (float)D + eps));
    for (int i = threadIdx.x; i < D; i += blockDim.x) yr[i] = (xr[i] * r) * w[i];
}

}  // namespace

hipError_t launch_embed(const void *E, const int32_t *tok, int64_t tok_ld, int M, int T,
                        const int *pos_dev, int pos0, const int *pos_rows, const int2 *rowmap, int D,
                        int dtype, void *x, hipStream_t s)
{
    int64_t row_bytes = (int64_t)D * (dtype == 1 ? 2 : 4);
    if (M <= 0) return hipSuccess;
    hipLaunchKernelGGL(embed_kernel, dim3(M), dim3(kThreads), 0, s, (const char *)E, tok,
                       tok_ld, T, pos_dev, pos0, pos_rows, rowmap, row_bytes, (char *)x);
    return hipGetLastError();
}

hipError_t launch_gather_rows(const void *x, const int *idx, int n, int D, int es, void *out, hipStream_t s)
{
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(gather_rows_kernel, dim3(n), dim3(kThreads), 0, s, (const char *)x, idx,
                       (int64_t)D * es, (char *)out);
    return hipGetLastError();
}

hipError_t launch_rmsnorm(const void *x, int64_t ldx, const void *w, int M, int D, float eps,
                          int dtype, void *y, hipStream_t s, int y_lay)
{
    if (M <= 0) return hipSuccess;
    if (y_lay && (dtype != 1 || D % 32)) return hipErrorInvalidValue;
    if ((y_lay == 1 || y_lay == 2) && M > 16 * y_lay) return hipErrorInvalidValue;
    if (dtype == 1 && D > 64 * 8 * RMS_VEC) return hipErrorInvalidValue;  // the fp16 kernels hold a row in registers
    if (dtype == 1 && M <= 64)
        hipLaunchKernelGGL(rmsnorm_row_kernel<0>, dim3(M), dim3(512), 0, s, (const half_t *)x, ldx,
                           (const half_t *)w, D, eps, (half_t *)y, y_lay, (const float *)nullptr, (half_t *)nullptr);
    else if (dtype == 1 && y_lay == ACT_TILED && D % 1024 == 0)
        // the output buffer spans whole 16-row groups
        hipLaunchKernelGGL(rmsnorm_tiled_kernel, dim3((M + 15) / 16 * 2), dim3(512), (size_t)10 * D, s,
                           (const half_t *)x, ldx, (const half_t *)w, M, D, eps, (half_t *)y);
    else if (dtype == 1)
        hipLaunchKernelGGL(rmsnorm_f16_kernel, dim3((M + 3) / 4), dim3(256), 0, s, (const half_t *)x, ldx,
                           (const half_t *)w, M, D, eps, (half_t *)y, y_lay);
    else
        hipLaunchKernelGGL(rmsnorm_f32_kernel, dim3(M), dim3(kThreads), 0, s, (const float *)x, ldx,
                           (const float *)w, D, eps, (float *)y);
    return hipGetLastError();
}

hipError_t launch_rmsnorm_resid(const float *part, int S, void *x, const void *w, int M, int D, float eps, void *y,
                                hipStream_t s, int y_lay)
{
    if (M <= 0) return hipSuccess;
    if (!part || S < 1 || M > 64 || D % 32 || D > 64 * 8 * RMS_VEC) return hipErrorInvalidValue;
    if ((y_lay == 1 || y_lay == 2) && M > 16 * y_lay) return hipErrorInvalidValue;
    if (S == 2)
        hipLaunchKernelGGL(rmsnorm_row_kernel<2>, dim3(M), dim3(512), 0, s, (const half_t *)x, (int64_t)D,
                           (const half_t *)w, D, eps, (half_t *)y, y_lay, part, (half_t *)x);
    else if (S == 4)
        hipLaunchKernelGGL(rmsnorm_row_kernel<4>, dim3(M), dim3(512), 0, s, (const half_t *)x, (int64_t)D,
                           (const half_t *)w, D, eps, (half_t *)y, y_lay, part, (half_t *)x);
    else
        return hipErrorInvalidValue;  // the products split K in two or four
    return hipGetLastError();
}
