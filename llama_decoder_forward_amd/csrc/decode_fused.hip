// One decoder layer of a one-row decode step in a single launch (walkthrough
// sections 3.5-3.7: attention_norm, wq|wk|wv with RoPE and the KV-cache
// write, attention, wo + residual, ffn_norm, w1|w3 with SwiGLU, w2 +
// residual).
//
// A one-row step streams every weight once and does almost no arithmetic, so
// the separate launches of the products each lose their start-up and tail
// (a few microseconds of half-empty HBM pipe per launch).  Here one
// persistent work-group per CU runs the five phases of the layer separated by
// grid barriers, and issues the first two weight rounds of the next phase
// before waiting at each barrier: the weight stream does not depend on the
// activations, so it keeps HBM busy while the barrier settles.  The attention
// phase runs on the first n_kv_heads work-groups; the others load their wo
// rows meanwhile.
//
// Every product, normalisation and epilogue here does the same arithmetic in
// the same order as the stand-alone kernels (two-stage RMSNorm sum, the
// wave-interleaved K split of the skinny product with its wave-ordered
// reduction, the decode attention of attn_decode.h), so the layer's output is
// bit-identical to the unfused launches.
//
// Data that one work-group writes and another reads inside the launch (q, the
// current position's K/V, the attention output, x, the SwiGLU output) is
// written and read with device-coherent accesses, which bypass the XCDs'
// private L2 caches; the barrier counts arrivals with relaxed device-scope
// atomics on eight group counters (work-groups by blockIdx % 8).  Every wait is
// bounded: after kSpinLimit polls the work-group raises the error flag and
// every later wait returns, so the launch always ends; the host reports the
// flag.
#include "common.h"
#include "attn_decode.h"

namespace {

constexpr int FNW = 8;         // waves per work-group
constexpr int FNT = FNW * 64;  // threads per work-group
constexpr int FU = 4;          // 1 KiB weight tiles per wave per round (as the one-row products)
static_assert(FU == 4, "wait_vm counts rounds of four loads");
constexpr int FROUND = FNW * FU;  // 32-wide K tiles per round of a 16-row block
constexpr unsigned kSpinLimit = 1u << 22;

__device__ __forceinline__ float r16(float x) { return (float)(half_t)x; }

__device__ __forceinline__ unsigned ld_agent(const unsigned *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Grid barrier number k (1, 2, ...) of this launch.  Every thread has waited
// for its own coherent stores (wait_vm) before; loads issued after those
// stay in flight across the barrier.  A work-group arrives with one atomic
// (no return, so it does not wait behind those loads) on the counter of its
// group (blockIdx % 8, one 128-byte line each); lanes 0..7 of wave 0 then
// poll the eight group counters until each has reached k times its group's
// size.
__device__ void grid_sync(unsigned *bar, unsigned *err, unsigned k)
{
    __syncthreads();
    if (threadIdx.x < 64) {
        const unsigned G = gridDim.x, lane = threadIdx.x;
        const unsigned ng = G < 8 ? G : 8;
        if (lane == 0)
            __hip_atomic_fetch_add(bar + 32 * (blockIdx.x & 7), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const unsigned target = lane < ng ? k * (G / 8 + (lane < G % 8 ? 1u : 0u)) : 0u;
        unsigned spins = 0;
        while (true) {
            const unsigned v = lane < ng ? ld_agent(bar + 32 * lane) : 0u;
            if (__all(v >= target)) break;
            if (__any(ld_agent(err) != 0u && lane == 0)) break;
            if (++spins > kSpinLimit) {
                if (lane == 0) __hip_atomic_store(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
    }
    __syncthreads();
}

// Wait until at most `pending` vector-memory operations of this wave are
// outstanding.  The counter retires in issue order, so issuing the coherent
// stores first and the next phase's weight loads after them, then waiting
// with pending = the number of those loads, completes the stores only.
__device__ __forceinline__ void wait_vm(int pending)
{
    if (pending >= 2 * FU) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    else if (pending >= FU) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// The work-group's share of one product: row blocks t = wg, wg + G, ... of a
// tiled matrix of NT blocks and KT 32-wide K tiles, against the staged
// activation row xs.  Work item j is round j % NR of the work-group's block
// j / NR; wave w's tiles in round r are K tiles r*FROUND + w*FU + u.  The
// weight stream is read with non-temporal loads.
struct Product {
    const half8 *W;
    int KT, NT, NR, n;  // K tiles, row blocks, rounds per block, this work-group's items
    int wg, G;
    __device__ Product(const half_t *w, int K, int N, int wg_, int G_)
        : W(reinterpret_cast<const half8 *>(w)), KT(K >> 5), NT(N >> 4), wg(wg_), G(G_)
    {
        NR = (KT + FROUND - 1) / FROUND;
        const int nb = wg < NT ? (NT - wg + G - 1) / G : 0;
        n = nb * NR;
    }
    __device__ __forceinline__ int block(int j) const { return wg + (j / NR) * G; }
    __device__ __forceinline__ void issue(int j, half8 (&buf)[FU], int wave, int lane) const
    {
        const int t = block(j), base = (j % NR) * FROUND + wave * FU;
        const half8 *src = W + (int64_t)t * KT * 64 + lane;
        if (base + FU <= KT) {  // a full round: no per-tile checks
#pragma unroll
            for (int u = 0; u < FU; u++) buf[u] = __builtin_nontemporal_load(src + (int64_t)(base + u) * 64);
        } else {  // the ragged last round: tiles past KT re-read the last one (zeroed when used)
#pragma unroll
            for (int u = 0; u < FU; u++) buf[u] = __builtin_nontemporal_load(src + (int64_t)min(base + u, KT - 1) * 64);
        }
    }
};

// Stage n8 half8 of src into xs (coherent loads when COH); with nw, RMS
// normalise the row as the stand-alone kernels do.
template <bool COH>
__device__ __forceinline__ void stage_row(const half_t *src, int K, const half_t *nw, float eps, half8 *xs,
                                          float *pss)
{
    const int tid = threadIdx.x, wave = tid >> 6;
    const int K8 = K >> 3;
    float ss = 0.f;
    for (int i = tid; i < K8; i += FNT) {
        half8 v = COH ? ld_coh_half8(src + 8 * i) : reinterpret_cast<const half8 *>(src)[i];
        xs[i] = v;
        if (nw) {
#pragma unroll
            for (int e = 0; e < 8; e++) { float f = (float)v[e]; ss += f * f; }
        }
    }
    if (nw) {
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
        if ((tid & 63) == 0) pss[wave] = ss;
    }
    __syncthreads();
    if (nw) {
#pragma clang fp contract(off)
        float t = 0.f;
        for (int ww = 0; ww < FNW; ww++) t += pss[ww];
        const float r = __frcp_rn(__fsqrt_rn(t / (float)K + eps));
        for (int i = tid; i < K8; i += FNT) {
            half8 v = xs[i], wv = reinterpret_cast<const half8 *>(nw)[i];
#pragma unroll
            for (int e = 0; e < 8; e++) {
                float n = (float)(half_t)((float)v[e] * r);
                v[e] = (half_t)(n * (float)wv[e]);
            }
            xs[i] = v;
        }
        __syncthreads();
    }
}

struct LayerArgs {
    const half_t *wqkv, *wo, *w13, *w2;  // packed, tiled
    const half_t *nw_attn, *nw_ffn;      // RMSNorm weights [D]
    half_t *kc, *vc;                     // this layer's cache
    KvPages pg;
    int S;                               // positions per cache stream
    const float *rope;                   // [S][hd/2][2]
    const int *pos;                      // the row's position (device memory)
    half_t *x;                           // residual row [D]
    half_t *q, *o, *g;                   // [H*hd], [H*hd], [F]
    unsigned *bar, *bar_reset, *err;     // this launch's eight group counters, the next launch's, error flag
    int D, H, Hkv, F;
    float eps;
};

template <bool PAGED>
__global__ __launch_bounds__(FNT, 1) void decode_layer_kernel(LayerArgs a)
{
#pragma clang fp contract(off)
    constexpr int hd = 128;
    extern __shared__ half8 xs[];  // the staged activation row
    __shared__ floatx4 red[2][FNW][64];
    __shared__ float pss[FNW];
    __shared__ floatx4 so[FNW][8][64];
    __shared__ float sm[FNW][16], sl[FNW][16];
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int mc = lane & 15, g = lane >> 4;
    const int wg = blockIdx.x, G = gridDim.x;
    const half8 z = {};
    const int pos = *a.pos;

    if (wg == 0 && tid < 8)  // the next launch's counters (its predecessor, this one, has ended by then)
        __hip_atomic_store(a.bar_reset + 32 * tid, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

    half8 A[FU], B[FU];
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};

    // items of product p, two rounds in flight; `epi(t, s)` runs on wave 0
    // with the reduced fragment of block t
    auto run = [&](const Product &p, auto epi) {
        auto compute = [&](int j, const half8 (&buf)[FU]) {
            const int r = j % p.NR, base = r * FROUND + wave * FU;
            if (r == 0) acc = floatx4{0.f, 0.f, 0.f, 0.f};
            if (base + FU <= p.KT) {
#pragma unroll
                for (int u = 0; u < FU; u++) {
                    half8 b0 = xs[(base + u) * 4 + g];
                    b0 = mc == 0 ? b0 : z;  // the one activation row is MFMA column 0
                    acc = adec::mfma16(buf[u], b0, acc);
                }
            } else {
#pragma unroll
                for (int u = 0; u < FU; u++) {
                    const bool ok = base + u < p.KT;
                    half8 b0 = xs[min(base + u, p.KT - 1) * 4 + g];
                    b0 = (ok && mc == 0) ? b0 : z;
                    acc = adec::mfma16(ok ? buf[u] : z, b0, acc);
                }
            }
            if (r == p.NR - 1) {
                const int par = (j / p.NR) & 1;
                red[par][wave][lane] = acc;
                __syncthreads();
                if (wave == 0) {
                    floatx4 s0 = red[par][0][lane];
                    for (int ww = 1; ww < FNW; ww++) s0 += red[par][ww][lane];
                    epi(p.block(j), s0);
                }
            }
        };
        // steady state: both buffers refilled every pass, so the loads in
        // flight at the top of the loop are always A's then B's
        int j = 0;
        for (; j + 3 < p.n; j += 2) {
            compute(j, A);
            p.issue(j + 2, A, wave, lane);
            compute(j + 1, B);
            p.issue(j + 3, B, wave, lane);
        }
        // the last one to three items
        if (j < p.n) {
            compute(j, A);
            if (j + 2 < p.n) p.issue(j + 2, A, wave, lane);
        }
        if (j + 1 < p.n) compute(j + 1, B);
        if (j + 2 < p.n) compute(j + 2, A);
    };
    // the first two items of p, issued ahead; returns the loads issued
    auto prefetch = [&](const Product &p) {
        if (p.n > 0) p.issue(0, A, wave, lane);
        if (p.n > 1) p.issue(1, B, wave, lane);
        return (p.n > 1 ? 2 : p.n) * FU;
    };

    const int qrows = a.H * hd, krows = a.Hkv * hd, HD = a.H * hd;
    const Product pqkv(a.wqkv, a.D, qrows + 2 * krows, wg, G);
    const Product po(a.wo, HD, a.D, wg, G);
    const Product p13(a.w13, a.D, 2 * a.F, wg, G);
    const Product p2(a.w2, a.F, a.D, wg, G);

    // ---- phase A: attention_norm, wq|wk|wv, RoPE, q and the KV write
    // x first: its wait would otherwise also wait for the weight loads
    stage_row<false>(a.x, a.D, a.nw_attn, a.eps, xs, pss);
    prefetch(pqkv);
    run(pqkv, [&](int t, floatx4 s) {
        const int n = t * 16 + 4 * g;
        if (mc != 0) return;
        if (n < qrows + krows) {
            const int d0 = n % hd;
            const float *cs = a.rope + ((int64_t)pos * (hd / 2) + d0 / 2) * 2;
            half4 o;
            #pragma unroll
            for (int p = 0; p < 2; p++) {
                float x0 = r16(s[2 * p]), x1 = r16(s[2 * p + 1]);
                float c = cs[2 * p], sn = cs[2 * p + 1];
                float re = x0 * c - x1 * sn;
                float im = x0 * sn + x1 * c;
                o[2 * p] = (half_t)re;
                o[2 * p + 1] = (half_t)im;
            }
            if (n < qrows) {
                st_coh_half4(a.q + n, o);
            } else {
                int off;
                const int64_t st = kv_stream(a.pg, 0, (n - qrows) / hd, pos, a.Hkv, off);
                st_coh_half4(a.kc + k_offset(st, off, d0, a.S, hd), o);
            }
        } else {
            const int rr = n - qrows - krows, d0 = rr % hd;
            int off;
            const int64_t st = kv_stream(a.pg, 0, rr / hd, pos, a.Hkv, off);
            half_t *vp = a.vc + v16_offset(st, off, d0, a.S, hd);
            #pragma unroll
            for (int i = 0; i < 4; i++) st_coh_half(vp + i * 32, (half_t)s[i]);
        }
    });
    wait_vm(wg >= a.Hkv ? prefetch(po) : 0);  // attention work-groups load theirs afterwards
    grid_sync(a.bar, a.err, 1);

    // ---- phase B: attention of the row's KV heads, one work-group each
    if (wg < a.Hkv) {
        adec::attn_decode_wg<FNW, false, PAGED, true>(a.q, a.kc, a.vc, a.H, a.Hkv, a.S, a.pg, 0, wg, pos + 1, a.o,
                                                      0, so, sm, sl);
        wait_vm(prefetch(po));
    }
    grid_sync(a.bar, a.err, 2);

    // ---- phase C: wo + residual
    stage_row<true>(a.o, HD, nullptr, 0.f, xs, pss);
    run(po, [&](int t, floatx4 s) {
        if (mc != 0) return;
        half_t *p = a.x + t * 16 + 4 * g;
        half4 r = *reinterpret_cast<const half4 *>(p), o;  // not yet written in this launch
        #pragma unroll
        for (int i = 0; i < 4; i++) o[i] = (half_t)((float)r[i] + r16(s[i]));
        st_coh_half4(p, o);
    });
    wait_vm(prefetch(p13));
    grid_sync(a.bar, a.err, 3);

    // ---- phase D: ffn_norm, w1|w3, SwiGLU
    stage_row<true>(a.x, a.D, a.nw_ffn, a.eps, xs, pss);
    run(p13, [&](int t, floatx4 s) {
        // rows 0..7 of block t are w1 rows 8t.., rows 8..15 the w3 rows:
        // lane groups 0/1 hold a, groups 2/3 the matching b
        float bv[4];
        #pragma unroll
        for (int i = 0; i < 4; i++) bv[i] = __shfl_xor(s[i], 32);
        if (mc != 0 || g >= 2) return;
        half4 o;
        #pragma unroll
        for (int i = 0; i < 4; i++) {
            float av = r16(s[i]);
            float sv = r16(av / (1.0f + expf(-av)));
            o[i] = (half_t)(sv * r16(bv[i]));
        }
        st_coh_half4(a.g + t * 8 + 4 * g, o);
    });
    wait_vm(prefetch(p2));
    grid_sync(a.bar, a.err, 4);

    // ---- phase E: w2 + residual
    stage_row<true>(a.g, a.F, nullptr, 0.f, xs, pss);
    run(p2, [&](int t, floatx4 s) {
        if (mc != 0) return;
        half_t *p = a.x + t * 16 + 4 * g;
        const half4 r = ld_coh_half4(p);  // written in phase C
        half4 o;
        #pragma unroll
        for (int i = 0; i < 4; i++) o[i] = (half_t)((float)r[i] + r16(s[i]));
        st_coh_half4(p, o);
    });
}

}  // namespace

// Dynamic LDS of the fused layer: the largest staged row.
static size_t fused_lds(int D, int HD, int F)
{
    int k = D > HD ? D : HD;
    k = k > F ? k : F;
    return (size_t)k * 2;
}

bool fused_layer_fits(int D, int H, int Hkv, int F, int G)
{
    // the attention phase needs a work-group per KV head; the staged row and
    // the fixed LDS must fit 160 KiB
    return Hkv <= G && fused_lds(D, H * 128, F) + 56 * 1024 <= 160 * 1024;
}

hipError_t launch_decode_layer(const FusedLayer &f, int G, hipStream_t s)
{
    LayerArgs a;
    a.wqkv = (const half_t *)f.wqkv; a.wo = (const half_t *)f.wo; a.w13 = (const half_t *)f.w13; a.w2 = (const half_t *)f.w2;
    a.nw_attn = (const half_t *)f.nw_attn; a.nw_ffn = (const half_t *)f.nw_ffn;
    a.kc = (half_t *)f.kc; a.vc = (half_t *)f.vc; a.pg = f.pg; a.S = f.S; a.rope = f.rope;
    a.pos = f.pos;
    a.x = (half_t *)f.x; a.q = (half_t *)f.q; a.o = (half_t *)f.o; a.g = (half_t *)f.g;
    a.bar = f.bar; a.bar_reset = f.bar_reset; a.err = f.err;
    a.D = f.D; a.H = f.H; a.Hkv = f.Hkv; a.F = f.F; a.eps = f.eps;
    if (!fused_layer_fits(f.D, f.H, f.Hkv, f.F, G)) return hipErrorInvalidValue;
    const size_t lds = fused_lds(f.D, f.H * 128, f.F);
    if (f.pg.tab)
        hipLaunchKernelGGL(decode_layer_kernel<true>, dim3(G), dim3(FNT), lds, s, a);
    else
        hipLaunchKernelGGL(decode_layer_kernel<false>, dim3(G), dim3(FNT), lds, s, a);
    return hipGetLastError();
}
