// Sampling from the last-position logits (walkthrough sections 4.2-4.3;
// course notes on generate, section 4): greedy argmax, temperature softmax,
// and top-p.
//
// Top-p is computed exactly so that it does not depend on reduction order:
// with tokens ranked by (P desc, id asc), Q_i = floor(P_i * 2^48) and E_i the
// sum of Q over tokens ranked above i, token i is kept iff E_i <= floor(p *
// 2^48); with S the kept mass and U = floor(u * 2^24), the draw is the kept
// token whose interval [E_i, E_i + Q_i) holds t = floor(U * S / 2^24).
//
// Instead of sorting, a radix select over the 32-bit patterns of P (which
// order like the values, P >= 0) finds the smallest probability value v with
// A(v) <= X, where A(v) is the mass of all tokens with P > v: with X = the
// threshold it gives the last kept value (and S), with X = t the drawn
// value.  Tokens of equal P occupy consecutive ranks in id order, each with
// the same Q, so the rank inside a tie group is an integer division, and the
// id is found by a counting pass in id order.
#include "common.h"

namespace {

constexpr int kSampThreads = 1024;

__device__ __forceinline__ uint64_t qmass(uint32_t pbits)
{
    return (uint64_t)((double)__uint_as_float(pbits) * 281474976710656.0);  // floor(P * 2^48)
}

// ---------------------------------------------------------------------------
// Greedy: argmax, lowest id among equal maxima.
// ---------------------------------------------------------------------------
__global__ void argmax_kernel(const float *logits, int V, int32_t *tok, int64_t tok_ld,
                              int write_col, int32_t *out)
{
    __shared__ float sv[16];
    __shared__ int si[16];
    const int b = blockIdx.x;
    const float *row = logits + (int64_t)b * V;
    float best = -INFINITY;
    int bi = 0x7fffffff;
    for (int i = threadIdx.x; i < V; i += blockDim.x) {
        float v = row[i];
        if (v > best || (v == best && i < bi)) { best = v; bi = i; }
    }
    for (int o = 32; o > 0; o >>= 1) {
        float ov = __shfl_xor(best, o);
        int oi = __shfl_xor(bi, o);
        if (ov > best || (ov == best && oi < bi)) { best = ov; bi = oi; }
    }
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) { sv[w] = best; si[w] = bi; }
    __syncthreads();
    if (threadIdx.x == 0) {
        best = sv[0];
        bi = si[0];
        for (int k = 1; k < (int)(blockDim.x >> 6); k++)
            if (sv[k] > best || (sv[k] == best && si[k] < bi)) { best = sv[k]; bi = si[k]; }
        if (bi < 0 || bi >= V) bi = 0;  // every logit NaN: keep the id in range
        if (write_col >= 0) tok[(int64_t)b * tok_ld + write_col] = bi;
        if (out) out[b] = bi;
    }
}

// ---------------------------------------------------------------------------
// P = softmax(logits / temperature) in fp32 with the maximum subtracted.
// ---------------------------------------------------------------------------
__device__ float block_max(float v, float *red)
{
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    float r = red[0];
    for (int k = 1; k < (int)(blockDim.x >> 6); k++) r = fmaxf(r, red[k]);
    return r;
}

__device__ float block_sumf(float v, float *red)
{
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    float r = 0.f;
    for (int k = 0; k < (int)(blockDim.x >> 6); k++) r += red[k];
    return r;
}

__global__ __launch_bounds__(kSampThreads) void softmax_temp_kernel(const float *logits, int V,
                                                                    float temperature, float *probs)
{
    __shared__ float red[kSampThreads / 64];
    const float *row = logits + (int64_t)blockIdx.x * V;
    float *pr = probs + (int64_t)blockIdx.x * V;
    float mx = -INFINITY;
    for (int i = threadIdx.x; i < V; i += blockDim.x) mx = fmaxf(mx, row[i] / temperature);
    mx = block_max(mx, red);
    float s = 0.f;
    for (int i = threadIdx.x; i < V; i += blockDim.x) {
        float e = expf(row[i] / temperature - mx);
        pr[i] = e;
        s += e;
    }
    s = block_sumf(s, red);
    for (int i = threadIdx.x; i < V; i += blockDim.x) pr[i] = pr[i] / s;
}

// ---------------------------------------------------------------------------
// Top-p
// ---------------------------------------------------------------------------
struct SelectResult {
    uint32_t key;    // bit pattern of the selected probability value
    uint64_t above;  // A(key): mass of all tokens with larger P
    uint32_t count;  // tokens with exactly this P
};

// Smallest present key v with A(v) <= X (one work-group, keys in global P).
__device__ SelectResult radix_select(const uint32_t *keys, int V, uint64_t X, uint32_t *hcnt,
                                     uint64_t *hsum, SelectResult *res)
{
    uint32_t prefix = 0, pmask = 0;
    uint64_t above = 0;
    uint32_t cnt_last = 0;
    for (int shift = 24; shift >= 0; shift -= 8) {
        for (int i = threadIdx.x; i < 256; i += blockDim.x) { hcnt[i] = 0; hsum[i] = 0; }
        __syncthreads();
        for (int i = threadIdx.x; i < V; i += blockDim.x) {
            uint32_t k = keys[i];
            if ((k & pmask) == prefix) {
                uint32_t d = (k >> shift) & 255u;
                atomicAdd(&hcnt[d], 1u);
                atomicAdd((unsigned long long *)&hsum[d], (unsigned long long)qmass(k));
            }
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            // G(d) = above + mass of buckets > d; pick the lowest present d
            // with G(d) <= X.
            uint64_t G = above;
            int pick = -1;
            uint64_t gpick = 0;
            for (int d = 255; d >= 0; d--) {
                if (hcnt[d] > 0 && G <= X) { pick = d; gpick = G; }
                G += hsum[d];
            }
            if (pick < 0) pick = 255;  // unreachable for X >= 0 (the top token has A = 0)
            res->key = prefix | ((uint32_t)pick << shift);
            res->above = gpick;
            res->count = hcnt[pick];
        }
        __syncthreads();
        prefix = res->key;
        pmask |= 255u << shift;
        above = res->above;
        cnt_last = res->count;
        __syncthreads();
    }
    SelectResult r;
    r.key = prefix;
    r.above = above;
    r.count = cnt_last;
    return r;
}

__global__ __launch_bounds__(kSampThreads) void top_p_kernel(const float *probs, int V, float top_p,
                                                             const float *uniforms, int32_t *tok,
                                                             int64_t tok_ld, int write_col,
                                                             int32_t *out)
{
    __shared__ uint32_t hcnt[256];
    __shared__ uint64_t hsum[256];
    __shared__ SelectResult res;
    __shared__ uint32_t scan[kSampThreads / 64];
    __shared__ int found;
    const int b = blockIdx.x;
    const uint32_t *keys = reinterpret_cast<const uint32_t *>(probs + (int64_t)b * V);

    const uint64_t thr = (uint64_t)floor((double)top_p * 281474976710656.0);
    SelectResult s1 = radix_select(keys, V, thr, hcnt, hsum, &res);
    const uint64_t q1 = qmass(s1.key);
    uint64_t kept = s1.count;
    if (q1 > 0) {
        uint64_t lim = (thr - s1.above) / q1 + 1;
        if (lim < kept) kept = lim;
    }
    const uint64_t S = s1.above + kept * q1;
    const uint64_t U = (uint64_t)floor((double)uniforms[b] * 16777216.0);
    const uint64_t lo = U * S, hi = __umul64hi(U, S);
    const uint64_t t = (lo >> 24) | (hi << 40);

    SelectResult s2 = radix_select(keys, V, t, hcnt, hsum, &res);
    const uint64_t q2 = qmass(s2.key);
    const uint32_t m = q2 > 0 ? (uint32_t)((t - s2.above) / q2) : 0u;

    // id of the m-th token (in id order) whose P bits equal s2.key
    const int per = (V + blockDim.x - 1) / blockDim.x;
    const int i0 = threadIdx.x * per, i1 = min(V, i0 + per);
    uint32_t c = 0;
    for (int i = i0; i < i1; i++) c += keys[i] == s2.key;
    // exclusive scan of c over the block
    uint32_t incl = c;
    for (int o = 1; o < 64; o <<= 1) {
        uint32_t v = __shfl_up(incl, o);
        if ((int)(threadIdx.x & 63) >= o) incl += v;
    }
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 63) scan[w] = incl;
    if (threadIdx.x == 0) found = -1;
    __syncthreads();
    uint32_t base = 0;
    for (int k = 0; k < w; k++) base += scan[k];
    uint32_t excl = base + incl - c;
    if (m >= excl && m < excl + c) {
        uint32_t need = m - excl;
        for (int i = i0; i < i1; i++)
            if (keys[i] == s2.key) {
                if (need == 0) { found = i; break; }
                need--;
            }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int id = found >= 0 ? found : 0;
        if (write_col >= 0) tok[(int64_t)b * tok_ld + write_col] = id;
        if (out) out[b] = id;
    }
}

__global__ void set_int_kernel(int *dst, int v) { *dst = v; }

__global__ void set_tokens_kernel(int32_t *tok, int64_t tok_ld, int B, int col, const int32_t *vals,
                                  const uint8_t *mask)
{
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= B) return;
    if (mask && !mask[b]) return;
    tok[(int64_t)b * tok_ld + col] = vals[b];
}

}  // namespace

hipError_t launch_argmax(const float *logits, int B, int V, int32_t *tok, int64_t tok_ld,
                         int write_col, int32_t *out, hipStream_t s)
{
    hipLaunchKernelGGL(argmax_kernel, dim3(B), dim3(1024), 0, s, logits, V, tok, tok_ld, write_col,
                       out);
    return hipGetLastError();
}

hipError_t launch_softmax_temp(const float *logits, int B, int V, float temperature, float *probs,
                               hipStream_t s)
{
    hipLaunchKernelGGL(softmax_temp_kernel, dim3(B), dim3(kSampThreads), 0, s, logits, V,
                       temperature, probs);
    return hipGetLastError();
}

hipError_t launch_top_p(const float *probs, int B, int V, float top_p, const float *uniforms,
                        int32_t *tok, int64_t tok_ld, int write_col, int32_t *out, hipStream_t s)
{
    hipLaunchKernelGGL(top_p_kernel, dim3(B), dim3(kSampThreads), 0, s, probs, V, top_p, uniforms,
                       tok, tok_ld, write_col, out);
    return hipGetLastError();
}

hipError_t launch_set_int(int *dst, int v, hipStream_t s)
{
    hipLaunchKernelGGL(set_int_kernel, dim3(1), dim3(1), 0, s, dst, v);
    return hipGetLastError();
}

hipError_t launch_set_tokens(int32_t *tok, int64_t tok_ld, int B, int col, const int32_t *vals,
                             const uint8_t *mask, hipStream_t s)
{
    hipLaunchKernelGGL(set_tokens_kernel, dim3((B + 63) / 64), dim3(64), 0, s, tok, tok_ld, B, col,
                       vals, mask);
    return hipGetLastError();
}
