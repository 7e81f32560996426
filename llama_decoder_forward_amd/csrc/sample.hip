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
#include <cmath>
#include <mutex>
#include <string>

#include "../../include/llm.h"
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
// token column a sampler writes for row b (-1: none)
__device__ __forceinline__ int sample_col(int b, int write_col, const int *col_rows, int64_t tok_ld)
{
    if (!col_rows) return write_col;
    const int c = col_rows[b] + 1;
    return c < tok_ld ? c : -1;
}

__global__ void argmax_kernel(const float *logits, int V, int32_t *tok, int64_t tok_ld,
                              int write_col, const int *col_rows, int32_t *out)
{
    __shared__ float sv[16];
    __shared__ int si[16];
    const int b = blockIdx.x;
    const float *row = logits + (int64_t)b * V;
    float best = -INFINITY;
    int bi = 0x7fffffff;
    auto consider = [&](float v, int i) {
        if (v > best || (v == best && i < bi)) { best = v; bi = i; }
    };
    if ((V & 3) == 0) {
        // 16-byte loads, several in flight per thread
        const float4 *r4 = reinterpret_cast<const float4 *>(row);
#pragma unroll 4
        for (int i = threadIdx.x; i < (V >> 2); i += blockDim.x) {
            const float4 v = r4[i];
            consider(v.x, 4 * i);
            consider(v.y, 4 * i + 1);
            consider(v.z, 4 * i + 2);
            consider(v.w, 4 * i + 3);
        }
    } else {
        for (int i = threadIdx.x; i < V; i += blockDim.x) consider(row[i], i);
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
        const int col = sample_col(b, write_col, col_rows, tok_ld);
        if (col >= 0) tok[(int64_t)b * tok_ld + col] = bi;
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

__device__ double block_sumd(double v, double *red)
{
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    double r = 0.0;
    for (int k = 0; k < (int)(blockDim.x >> 6); k++) r += red[k];
    return r;
}

// One term of the temperature softmax: exp of the max-subtracted scaled
// logit d (fp32), evaluated in double and rounded once to fp32, so that it is
// the correctly rounded value (up to a double-rounding tie) on any machine.
__device__ __forceinline__ float softmax_term(float d) { return (float)exp((double)d); }

__global__ __launch_bounds__(kSampThreads) void softmax_temp_kernel(const float *logits, int V,
                                                                    float temperature, float *probs)
{
    __shared__ float red[kSampThreads / 64];
    __shared__ double redd[kSampThreads / 64];
    const float *row = logits + (int64_t)blockIdx.x * V;
    float *pr = probs + (int64_t)blockIdx.x * V;
    float mx = -INFINITY;
    for (int i = threadIdx.x; i < V; i += blockDim.x) mx = fmaxf(mx, row[i] / temperature);
    mx = block_max(mx, red);
    // the normaliser: the exact sum of the fp32 terms (accumulated in
    // double, whose error over V terms is far below one fp32 step), rounded
    // once to fp32
    double sd = 0.0;
    for (int i = threadIdx.x; i < V; i += blockDim.x) {
        const float e = softmax_term(row[i] / temperature - mx);
        pr[i] = e;
        sd += (double)e;
    }
    const float s = (float)block_sumd(sd, redd);
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
                                                             const int *col_rows, int32_t *out)
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
        const int col = sample_col(b, write_col, col_rows, tok_ld);
        if (col >= 0) tok[(int64_t)b * tok_ld + col] = id;
        if (out) out[b] = id;
    }
}

// ---------------------------------------------------------------------------
// Top-p for vocabularies of up to TP_MAXV tokens: one work-group per row with
// the row's probability patterns resident in LDS (computed there from the
// logits when the temperature softmax is fused in, with the arithmetic of
// softmax_temp_kernel: divisions by t and by the normaliser, terms and
// normaliser rounded once from double, so the probabilities do not depend
// on the order of the sum).  Same definition and result as top_p_kernel; the
// radix select runs in three passes over 11, 10 and 10 bits of the pattern
// (bit 31 is zero for P >= 0), fine enough that few tokens share a bucket,
// and the bucket scans are block-parallel instead of one thread's loop.
// ---------------------------------------------------------------------------
constexpr int TP_MAXV = 32768;
constexpr int TP_NB = 2048;

// floor(P * 2^48) from the pattern, in integers: P = m * 2^(e - 150) with the
// 24-bit significand m (e = 0: subnormal, no hidden bit, exponent of e = 1).
// The product in qmass() is exact in double, so the two agree.
__device__ __forceinline__ uint64_t qmass_bits(uint32_t k)
{
    const int e = (int)(k >> 23);
    const uint64_t m = e ? (uint64_t)((k & 0x7fffffu) | 0x800000u) : (uint64_t)(k & 0x7fffffu);
    const int ee = e ? e : 1;
    if (ee >= 102) return m << min(ee - 102, 39);  // P <= 1 keeps the shift <= 25
    return 102 - ee < 64 ? m >> (102 - ee) : 0;

}

struct TpShared {
    uint32_t hcnt[TP_NB];
    uint64_t hsum[TP_NB];
    uint32_t wcnt[kSampThreads / 64];
    float wf[kSampThreads / 64];
    double wd[kSampThreads / 64];
    SelectResult res;
    int found;
};



// Smallest present key v with A(v) <= X over the LDS keys (as radix_select).
__device__ __forceinline__ SelectResult radix_select_lds(const uint32_t *keys, int V, uint64_t X, TpShared &sh)
{
    uint32_t prefix = 0, pmask = 0;
    uint64_t above = 0;
    uint32_t cnt_last = 0;
    for (int ps = 0; ps < 3; ps++) {
        const int shift = ps == 0 ? 20 : (ps == 1 ? 10 : 0);
        const int nb = ps == 0 ? 2048 : 1024;
        for (int i = threadIdx.x; i < nb; i += blockDim.x) { sh.hcnt[i] = 0; sh.hsum[i] = 0; }
        __syncthreads();
        // four patterns per LDS read (V % 4 == 0)
        const uint4 *k4 = reinterpret_cast<const uint4 *>(keys);
        for (int i = threadIdx.x; i < V / 4; i += blockDim.x) {
            const uint4 q4 = k4[i];
            const uint32_t kk[4] = {q4.x, q4.y, q4.z, q4.w};
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const uint32_t k = kk[j];
                if ((k & pmask) == prefix) {
                    const uint32_t dg = (k >> shift) & (uint32_t)(nb - 1);
                    atomicAdd(&sh.hcnt[dg], 1u);
                    atomicAdd((unsigned long long *)&sh.hsum[dg], (unsigned long long)qmass_bits(k));
                }
            }
        }
        __syncthreads();
        // one wave scans the buckets: lane l owns [l*per, l*per + per), and
        // G(d) = above + mass of buckets > d
        if (threadIdx.x < 64) {
            const int lane = threadIdx.x, per = nb / 64, d0 = lane * per;
            uint64_t mine = 0;
            for (int j = 0; j < per; j++) mine += sh.hsum[d0 + j];
            uint64_t incl = mine;  // inclusive suffix over lanes
            for (int o = 1; o < 64; o <<= 1) {
                const uint64_t u = __shfl_down(incl, o);
                if (lane + o < 64) incl += u;
            }
            uint64_t G = above + (incl - mine);
            int cand = 0x7fffffff;
            uint64_t gc = 0;
            for (int j = per - 1; j >= 0; j--) {  // descending d, G grows
                const int dd = d0 + j;
                if (sh.hcnt[dd] > 0 && G <= X) { cand = dd; gc = G; }
                G += sh.hsum[dd];
            }
            int pick = cand;  // exists: the highest present bucket has G = above <= X
            for (int o = 32; o > 0; o >>= 1) pick = min(pick, __shfl_xor(pick, o));
            if (cand == pick) {
                sh.res.key = prefix | ((uint32_t)pick << shift);
                sh.res.above = gc;
                sh.res.count = sh.hcnt[pick];
            }
        }
        __syncthreads();
        prefix = sh.res.key;
        pmask |= (uint32_t)(nb - 1) << shift;
        above = sh.res.above;
        cnt_last = sh.res.count;
        __syncthreads();
    }
    SelectResult r;
    r.key = prefix;
    r.above = above;
    r.count = cnt_last;
    return r;
}

__global__ __launch_bounds__(kSampThreads) void top_p_lds_kernel(const float *src, int from_logits,
                                                                 float temperature, int V, float top_p,
                                                                 const float *uniforms, int32_t *tok,
                                                                 int64_t tok_ld, int write_col,
                                                                 const int *col_rows, int32_t *out)
{
    __shared__ TpShared sh;
    extern __shared__ uint32_t keys[];  // V patterns
    const int b = blockIdx.x;
    const float *row = src + (int64_t)b * V;
    if (from_logits) {
        // P = softmax(logits / t) in fp32 with the maximum subtracted, the
        // scaling and the normalisation as divisions (as softmax_temp_kernel)
        const float4 *r4 = reinterpret_cast<const float4 *>(row);
        float mx = -INFINITY;
        for (int i = threadIdx.x; i < V / 4; i += blockDim.x) {
            const float4 v = r4[i];
            mx = fmaxf(mx, fmaxf(fmaxf(v.x / temperature, v.y / temperature),
                                 fmaxf(v.z / temperature, v.w / temperature)));
        }
        mx = block_max(mx, sh.wf);
        double sd = 0.0;
        uint4 *k4 = reinterpret_cast<uint4 *>(keys);
        for (int i = threadIdx.x; i < V / 4; i += blockDim.x) {
            const float4 v = r4[i];
            const float e0 = softmax_term(v.x / temperature - mx), e1 = softmax_term(v.y / temperature - mx);
            const float e2 = softmax_term(v.z / temperature - mx), e3 = softmax_term(v.w / temperature - mx);
            k4[i] = make_uint4(__float_as_uint(e0), __float_as_uint(e1), __float_as_uint(e2), __float_as_uint(e3));
            sd += ((double)e0 + (double)e1) + ((double)e2 + (double)e3);
        }
        const float s = (float)block_sumd(sd, sh.wd);
        for (int i = threadIdx.x; i < V / 4; i += blockDim.x) {
            uint4 k = k4[i];
            k.x = __float_as_uint(__uint_as_float(k.x) / s) & 0x7fffffffu;
            k.y = __float_as_uint(__uint_as_float(k.y) / s) & 0x7fffffffu;
            k.z = __float_as_uint(__uint_as_float(k.z) / s) & 0x7fffffffu;
            k.w = __float_as_uint(__uint_as_float(k.w) / s) & 0x7fffffffu;
            k4[i] = k;
        }
    } else {
        for (int i = threadIdx.x; i < V; i += blockDim.x) keys[i] = __float_as_uint(row[i]) & 0x7fffffffu;
    }
    __syncthreads();

    const uint64_t thr = (uint64_t)floor((double)top_p * 281474976710656.0);
    const SelectResult s1 = radix_select_lds(keys, V, thr, sh);
    const uint64_t q1 = qmass_bits(s1.key);
    uint64_t kept = s1.count;
    if (q1 > 0) {
        const uint64_t lim = (thr - s1.above) / q1 + 1;
        if (lim < kept) kept = lim;
    }
    const uint64_t S = s1.above + kept * q1;
    const uint64_t U = (uint64_t)floor((double)uniforms[b] * 16777216.0);
    const uint64_t lo = U * S, hi = __umul64hi(U, S);
    const uint64_t t = (lo >> 24) | (hi << 40);

    const SelectResult s2 = radix_select_lds(keys, V, t, sh);
    const uint64_t q2 = qmass_bits(s2.key);
    const uint32_t m = q2 > 0 ? (uint32_t)((t - s2.above) / q2) : 0u;

    // id of the m-th token (in id order) whose pattern equals s2.key: wave w
    // owns ids [w*chunk, (w+1)*chunk), lanes read consecutive patterns (no
    // LDS bank conflicts) and count matches with ballots
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
    const int chunk = (V + nw * 64 - 1) / (nw * 64) * 64;
    const int w0 = w * chunk, w1 = min(V, w0 + chunk);
    uint32_t c = 0;
    for (int base = w0; base < w1; base += 64) {
        const int i = base + lane;
        c += (uint32_t)__popcll(__ballot(i < w1 && keys[i] == s2.key));
    }
    if (lane == 0) sh.wcnt[w] = c;
    if (threadIdx.x == 0) sh.found = -1;
    __syncthreads();
    uint32_t excl = 0;
    for (int k = 0; k < w; k++) excl += sh.wcnt[k];
    if (m >= excl && m < excl + c) {  // wave-uniform
        uint32_t need = m - excl;
        for (int base = w0; base < w1; base += 64) {
            const int i = base + lane;
            uint64_t bal = __ballot(i < w1 && keys[i] == s2.key);
            const uint32_t n = (uint32_t)__popcll(bal);
            if (need < n) {
                for (uint32_t j = 0; j < need; j++) bal &= bal - 1;  // drop the lowest set bits
                if (lane == 0) sh.found = base + (int)__builtin_ctzll(bal);
                break;
            }
            need -= n;
        }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        const int id = sh.found >= 0 ? sh.found : 0;
        const int col = sample_col(b, write_col, col_rows, tok_ld);
        if (col >= 0) tok[(int64_t)b * tok_ld + col] = id;
        if (out) out[b] = id;
    }
}

__global__ void set_int_kernel(int *dst, int v) { *dst = v; }

__global__ void inc_ints_kernel(int *dst, int n)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) dst[i] += 1;
}

__global__ void set_tokens_rows_kernel(int32_t *tok, int64_t tok_ld, int B, const int *col_rows,
                                       const int32_t *vals, const uint8_t *mask)
{
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= B || (mask && !mask[b])) return;
    const int c = col_rows[b] + 1;
    if (c < tok_ld) tok[(int64_t)b * tok_ld + c] = vals[b];
}

__global__ void scatter_tokens_kernel(int32_t *tok, int64_t tok_ld, int M, const int2 *rowmap,
                                      const int32_t *vals)
{
    const int m = blockIdx.x * blockDim.x + threadIdx.x;
    if (m >= M) return;
    const int2 r = rowmap[m];
    tok[(int64_t)r.x * tok_ld + r.y] = vals[m];
}

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
                         int write_col, const int *col_rows, int32_t *out, hipStream_t s)
{
    hipLaunchKernelGGL(argmax_kernel, dim3(B), dim3(1024), 0, s, logits, V, tok, tok_ld, write_col,
                       col_rows, out);
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
                        int32_t *tok, int64_t tok_ld, int write_col, const int *col_rows, int32_t *out,
                        hipStream_t s)
{
    hipLaunchKernelGGL(top_p_kernel, dim3(B), dim3(kSampThreads), 0, s, probs, V, top_p, uniforms,
                       tok, tok_ld, write_col, col_rows, out);
    return hipGetLastError();
}

hipError_t launch_sample_top_p(const float *src, bool from_logits, float temperature, int B, int V, float top_p,
                               const float *uniforms, int32_t *tok, int64_t tok_ld, int write_col,
                               const int *col_rows, int32_t *out, float *probs_scratch, hipStream_t s)
{
    if (V <= TP_MAXV && V % 4 == 0) {
        hipLaunchKernelGGL(top_p_lds_kernel, dim3(B), dim3(kSampThreads), (size_t)V * 4, s, src, (int)from_logits,
                           temperature, V, top_p, uniforms, tok, tok_ld, write_col, col_rows, out);
        return hipGetLastError();
    }
    const float *probs = src;
    if (from_logits) {
        hipError_t e = launch_softmax_temp(src, B, V, temperature, probs_scratch, s);
        if (e != hipSuccess) return e;
        probs = probs_scratch;
    }
    return launch_top_p(probs, B, V, top_p, uniforms, tok, tok_ld, write_col, col_rows, out, s);
}

hipError_t launch_set_int(int *dst, int v, hipStream_t s)
{
    hipLaunchKernelGGL(set_int_kernel, dim3(1), dim3(1), 0, s, dst, v);
    return hipGetLastError();
}

hipError_t launch_inc_ints(int *dst, int n, hipStream_t s)
{
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(inc_ints_kernel, dim3((n + 63) / 64), dim3(64), 0, s, dst, n);
    return hipGetLastError();
}

hipError_t launch_set_tokens_rows(int32_t *tok, int64_t tok_ld, int B, const int *col_rows, const int32_t *vals,
                                  const uint8_t *mask, hipStream_t s)
{
    hipLaunchKernelGGL(set_tokens_rows_kernel, dim3((B + 63) / 64), dim3(64), 0, s, tok, tok_ld, B, col_rows, vals,
                       mask);
    return hipGetLastError();
}

hipError_t launch_scatter_tokens(int32_t *tok, int64_t tok_ld, int M, const int2 *rowmap, const int32_t *vals,
                                 hipStream_t s)
{
    if (M <= 0) return hipSuccess;
    hipLaunchKernelGGL(scatter_tokens_kernel, dim3((M + 255) / 256), dim3(256), 0, s, tok, tok_ld, M, rowmap, vals);
    return hipGetLastError();
}

hipError_t launch_set_tokens(int32_t *tok, int64_t tok_ld, int B, int col, const int32_t *vals,
                             const uint8_t *mask, hipStream_t s)
{
    hipLaunchKernelGGL(set_tokens_kernel, dim3((B + 63) / 64), dim3(64), 0, s, tok, tok_ld, B, col,
                       vals, mask);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Sampling without allocation, for callers that cannot allocate device
// memory.  The probability rows of the two-launch path live in a file-scope
// device array instead of a handle's buffer.  Host code never uses the
// array's name as an address: the address is looked up once per device with
// hipGetSymbolAddress and passed to the kernels.
// ---------------------------------------------------------------------------
namespace {

constexpr int64_t kStaticProbFloats = (int64_t)1 << 22;  // 16 MiB: B * V floats
constexpr int kMaxDevices = 64;

static __device__ __align__(256) float scratch[kStaticProbFloats];

std::mutex g_scratch_mu;
float *g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch` (NULL on error).
float *static_scratch(hipError_t *err)
{
    int dev = 0;
    *err = hipGetDevice(&dev);
    if (*err != hipSuccess) return nullptr;
    if (dev < 0 || dev >= kMaxDevices) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        *err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (*err != hipSuccess) return nullptr;
        g_scratch_ptr[dev] = (float *)ptr;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

static thread_local std::string g_static_err;

static int static_fail(int code, const char *msg)
{
    g_static_err = msg;
    return code;
}

const char *static_call_error() { return g_static_err.c_str(); }

extern "C" int llm_sample_logits_static(const float *logits_d, int32_t B, int32_t V, float temperature,
                                        float top_p, const float *uniforms_d, int32_t *out_d,
                                        void *hip_stream)
{
    g_static_err.clear();
    if (!logits_d || !out_d) return static_fail(LLM_EINVAL, "logits and out must not be NULL");
    if (B < 1 || V < 2 || V > (1 << 22)) return static_fail(LLM_EINVAL, "need B >= 1 and 2 <= V <= 2^22");
    if (!std::isfinite(temperature)) return static_fail(LLM_EINVAL, "temperature must be finite");
    hipStream_t s = (hipStream_t)hip_stream;
    hipError_t e;
    if (temperature <= 0.f) {
        e = launch_argmax(logits_d, B, V, nullptr, 0, -1, nullptr, out_d, s);
        return e == hipSuccess ? LLM_OK : static_fail(LLM_EDEVICE, hipGetErrorString(e));
    }
    if (!(top_p > 0.f && top_p <= 1.f)) return static_fail(LLM_EINVAL, "top_p must be in (0, 1]");
    if (!uniforms_d) return static_fail(LLM_EINVAL, "uniforms are required when temperature > 0");
    float *probs = nullptr;
    if (!(V <= TP_MAXV && V % 4 == 0)) {  // the two-launch path stages B x V probabilities
        if ((int64_t)B * V > kStaticProbFloats)
            return static_fail(LLM_EINVAL, "B * V exceeds the static probability buffer (4194304 floats)");
        probs = static_scratch(&e);
        if (!probs) return static_fail(LLM_EDEVICE, hipGetErrorString(e));
    }
    e = launch_sample_top_p(logits_d, true, temperature, B, V, top_p, uniforms_d, nullptr, 0, -1, nullptr, out_d,
                            probs, s);
    return e == hipSuccess ? LLM_OK : static_fail(LLM_EDEVICE, hipGetErrorString(e));
}
