// Seeded weight generation on the device, fills and weight read-back.
//
// Weights come from SplitMix64 (Steele, Lea & Flood, OOPSLA 2014): output n
// of the generator started at state s is mix(s + (n+1) * gamma).  Tensor t of
// a model with seed S draws from the stream whose state is output t of the
// generator started at S; logical element e (row-major over [out][in]) takes
// output e of that stream.  Its four 16-bit fields are summed (Irwin-Hall,
// n = 4), centred, scaled to standard deviation 0.02 in double precision and
// rounded once to the storage type.  Tensor ids: 0 embedding, 1 output head,
// 16 + 8*layer + {0 wq, 1 wk, 2 wv, 3 wo, 4 w1, 5 w2, 6 w3}.
#include "common.h"

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;
constexpr double kScale = 0x1.1bc779ef0d4e8p-21;  // nearest double to 0.02*sqrt(3)/65536

__device__ __forceinline__ uint64_t mix64(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

__device__ __forceinline__ double weight_at(uint64_t stream, uint64_t e)
{
    uint64_t h = mix64(stream + (e + 1) * kGamma);
    int64_t s = (int64_t)(h & 0xffff) + (int64_t)((h >> 16) & 0xffff) +
                (int64_t)((h >> 32) & 0xffff) + (int64_t)(h >> 48);
    return (double)(s - 131070) * kScale;
}

// binary16 round-to-nearest-even of a double, by integer manipulation of the
// double's fields (sign, 11-bit exponent, 52-bit fraction).
__device__ __forceinline__ uint16_t f64_to_f16_bits(double v)
{
    uint64_t b = (uint64_t)__double_as_longlong(v);
    uint32_t sign = (uint32_t)(b >> 48) & 0x8000u;
    int ex = (int)((b >> 52) & 0x7ff);
    uint64_t frac = b & ((1ull << 52) - 1);
    if (ex == 0x7ff) return (uint16_t)(sign | (frac ? 0x7e00u : 0x7c00u));
    if (ex == 0) return (uint16_t)sign;          // zero or far below the half range
    int e = ex - 1023;
    if (e > 15) return (uint16_t)(sign | 0x7c00u);
    uint64_t sig = frac | (1ull << 52);          // value = sig * 2^(e-52)
    int E = e < -14 ? -14 : e;                   // half exponent (subnormals share -14)
    int sh = 42 + E - e;                         // quantum 2^(E-10) = 2^(e-52) * 2^sh
    if (sh >= 54) return (uint16_t)sign;         // below half the smallest subnormal
    uint64_t q = sig >> sh;
    uint64_t rem = sig & ((1ull << sh) - 1);
    uint64_t halfway = 1ull << (sh - 1);
    if (rem > halfway || (rem == halfway && (q & 1))) q++;
    if (E == -14 && q < 1024) return (uint16_t)(sign | (uint32_t)q);
    if (q == 2048) { q = 1024; E++; }
    if (E > 15) return (uint16_t)(sign | 0x7c00u);
    return (uint16_t)(sign | (uint32_t)((E + 15) << 10) | (uint32_t)(q - 1024));
}

// Logical tensor and row behind stored row n of a packed matrix.
struct Src { int tid; int64_t row; };

__device__ __forceinline__ Src packed_row_source(int mat, int layer, int64_t n, int H, int Hkv,
                                                 int hd)
{
    int base = 16 + 8 * layer;
    switch (mat) {
    case MAT_QKV:
        if (n < (int64_t)H * hd) return {base + 0, n};
        if (n < (int64_t)(H + Hkv) * hd) return {base + 1, n - (int64_t)H * hd};
        return {base + 2, n - (int64_t)(H + Hkv) * hd};
    case MAT_O: return {base + 3, n};
    case MAT_W13: {
        int64_t j = n >> 4, r = n & 15;
        return r < 8 ? Src{base + 4, 8 * j + r} : Src{base + 6, 8 * j + r - 8};
    }
    case MAT_W2: return {base + 5, n};
    case MAT_HEAD: return {1, n};
    default: return {0, n};  // embedding
    }
}

__device__ __forceinline__ uint64_t stream_of(uint64_t seed, int tid)
{
    return mix64(seed + ((uint64_t)tid + 1) * kGamma);
}

// One thread writes 8 consecutive stored halves.
__global__ void gen_f16_kernel(half_t *dst, int mat, int64_t N, int64_t K, uint64_t seed,
                               int layer, int H, int Hkv, int hd, int tiled)
{
    int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    int64_t groups = N * K / 8;
    if (g >= groups) return;
    int64_t n, k0;
    if (tiled) {
        int64_t tile = g >> 6, lane = g & 63, KT = K >> 5;
        n = (tile / KT) * 16 + (lane & 15);
        k0 = (tile % KT) * 32 + 8 * (lane >> 4);
    } else {
        n = (g * 8) / K;
        k0 = (g * 8) % K;
    }
    Src s = packed_row_source(mat, layer, n, H, Hkv, hd);
    uint64_t st = stream_of(seed, s.tid);
    uint16_t v[8];
#pragma unroll
    for (int e = 0; e < 8; e++) v[e] = f64_to_f16_bits(weight_at(st, (uint64_t)(s.row * K + k0 + e)));
    uint4 pk;
    pk.x = v[0] | ((uint32_t)v[1] << 16);
    pk.y = v[2] | ((uint32_t)v[3] << 16);
    pk.z = v[4] | ((uint32_t)v[5] << 16);
    pk.w = v[6] | ((uint32_t)v[7] << 16);
    reinterpret_cast<uint4 *>(dst)[g] = pk;
}

__global__ void gen_f32_kernel(float *dst, int mat, int64_t N, int64_t K, uint64_t seed, int layer,
                               int H, int Hkv, int hd)
{
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= N * K) return;
    int64_t n = i / K, k = i % K;
    Src s = packed_row_source(mat, layer, n, H, Hkv, hd);
    dst[i] = (float)weight_at(stream_of(seed, s.tid), (uint64_t)(s.row * K + k));
}

__global__ void fill_f16_kernel(half_t *dst, int64_t n, float v)
{
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = (half_t)v;
}

__global__ void fill_f32_kernel(float *dst, int64_t n, float v)
{
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = v;
}

__global__ void zero_kernel(uint4 *dst, int64_t n16, unsigned char *tail, int64_t ntail)
{
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t j = i; j < n16; j += stride) dst[j] = make_uint4(0, 0, 0, 0);
    if (i < ntail) tail[i] = 0;
}

// Logical element e of tensor `which` -> stored offset in the packed matrix.
__global__ void read_weights_kernel(const void *src, int dtype, int mat, int64_t Kp, int which,
                                    int H, int Hkv, int hd, int64_t Klog, int64_t first,
                                    int64_t count, void *out, int tiled)
{
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= count) return;
    int64_t e = first + i, row = e / Klog, col = e % Klog, n = row;
    if (mat == MAT_QKV) n = row + (which == 0 ? 0 : which == 1 ? (int64_t)H * hd : (int64_t)(H + Hkv) * hd);
    else if (mat == MAT_W13) n = (row >> 3) * 16 + (row & 7) + (which == 6 ? 8 : 0);
    int64_t off = tiled ? tiled_offset(n, col, Kp) : n * Kp + col;
    if (dtype == 1) ((uint16_t *)out)[i] = ((const uint16_t *)src)[off];
    else ((float *)out)[i] = ((const float *)src)[off];
}

inline unsigned blocks_for(int64_t n, int t) { return (unsigned)((n + t - 1) / t); }

}  // namespace

hipError_t launch_gen_weights_f16(half_t *dst, int mat, int64_t N, int64_t K, uint64_t seed,
                                  int layer, int H, int Hkv, int hd, int F, bool tiled,
                                  hipStream_t s)
{
    (void)F;
    int64_t groups = N * K / 8;
    hipLaunchKernelGGL(gen_f16_kernel, dim3(blocks_for(groups, 256)), dim3(256), 0, s, dst, mat, N,
                       K, seed, layer, H, Hkv, hd, tiled ? 1 : 0);
    return hipGetLastError();
}

hipError_t launch_gen_weights_f32(float *dst, int mat, int64_t N, int64_t K, uint64_t seed,
                                  int layer, int H, int Hkv, int hd, int F, hipStream_t s)
{
    (void)F;
    hipLaunchKernelGGL(gen_f32_kernel, dim3(blocks_for(N * K, 256)), dim3(256), 0, s, dst, mat, N,
                       K, seed, layer, H, Hkv, hd);
    return hipGetLastError();
}

hipError_t launch_fill_f16(half_t *dst, int64_t n, float v, hipStream_t s)
{
    hipLaunchKernelGGL(fill_f16_kernel, dim3(blocks_for(n, 256)), dim3(256), 0, s, dst, n, v);
    return hipGetLastError();
}

hipError_t launch_fill_f32(float *dst, int64_t n, float v, hipStream_t s)
{
    hipLaunchKernelGGL(fill_f32_kernel, dim3(blocks_for(n, 256)), dim3(256), 0, s, dst, n, v);
    return hipGetLastError();
}

hipError_t launch_zero_bytes(void *dst, int64_t bytes, hipStream_t s)
{
    if (bytes <= 0) return hipSuccess;
    int64_t n16 = bytes / 16, ntail = bytes % 16;
    unsigned char *tail = (unsigned char *)dst + n16 * 16;
    int64_t work = n16 > ntail ? n16 : ntail;
    unsigned blocks = blocks_for(work, 256);
    if (blocks > 65536u) blocks = 65536u;
    hipLaunchKernelGGL(zero_kernel, dim3(blocks), dim3(256), 0, s, (uint4 *)dst, n16, tail, ntail);
    return hipGetLastError();
}

hipError_t launch_read_weights(const void *src, int dtype, int mat, int64_t N, int64_t K,
                               int which, int H, int Hkv, int hd, int F, int64_t first,
                               int64_t count, void *out, hipStream_t s)
{
    (void)N;
    (void)F;
    int64_t Klog = K;
    int tiled = (dtype == 1 && mat != 5) ? 1 : 0;
    hipLaunchKernelGGL(read_weights_kernel, dim3(blocks_for(count, 256)), dim3(256), 0, s, src,
                       dtype, mat, K, which, H, Hkv, hd, Klog, first, count, out, tiled);
    return hipGetLastError();
}
