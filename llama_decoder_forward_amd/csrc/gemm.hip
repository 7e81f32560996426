// Linear layers of the decoder: Y = W X with fused epilogues.
//
// All projections of the layer (wq/wk/wv, wo, w1/w3, w2; walkthrough
// sections 3.5-3.6) and the output head are bias-free matrix products with
// fp32 accumulation, rounded once to fp16.  Their epilogues fuse the next
// elementwise step of the layer: RoPE plus the KV-cache write after the QKV
// projection (sections 3.3 and 3.5), the residual add after wo and w2
// (section 3.7), silu(w1 x) * w3 x after the gate/up projection (section
// 3.6), and the fp32 promotion of the logits (section 2).
//
// fp16 path: weights are tiled (see common.h) so that each lane's 16-byte
// load is an A operand of v_mfma_f32_16x16x32_f16; the activation rows are
// the B operand (column m = lane % 16).  The accumulator fragment of a lane
// holds rows n0 + 4*(lane/16) + i, i = 0..3, of column m.
#include "common.h"

namespace {

__device__ __forceinline__ floatx4 mfma16(half8 a, half8 b, floatx4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float r16(float x) { return (float)(half_t)x; }

// Apply the epilogue to one accumulator fragment.  Every lane of the wave
// must call this together (EP_SWIGLU exchanges values between lanes);
// `valid` masks the stores of lanes whose column is past M or whose rows are
// past N.
// KIND >= 0 fixes the epilogue kind at compile time (large kernels that
// apply it to many fragments keep only that kind's code).
template <int KIND = -1>
__device__ __forceinline__ void epilogue_frag(const Epilogue &ep, int n0, int m, bool valid,
                                              floatx4 acc, int lane)
{
#pragma clang fp contract(off)
    const int g = lane >> 4;
    const int n = n0 + 4 * g;
    switch (KIND >= 0 ? KIND : ep.kind) {
    case EP_STORE: {
        if (!valid) break;
        half4 o;
        for (int i = 0; i < 4; i++) o[i] = (half_t)acc[i];
        *reinterpret_cast<half4 *>((half_t *)ep.out + (int64_t)m * ep.ldo + n) = o;
        break;
    }
    case EP_LOGITS: {
        // the position a captured decode step reads moves to the next step
        // (every earlier kernel of the step has read it)
        if (ep.pos_advance && n0 == 0 && m == 0 && lane == 0) *ep.pos_advance += 1;
        if (!valid) break;
        float4 o = make_float4(r16(acc[0]), r16(acc[1]), r16(acc[2]), r16(acc[3]));
        *reinterpret_cast<float4 *>((float *)ep.out + (int64_t)m * ep.ldo + n) = o;
        break;
    }
    case EP_RESID: {
        if (!valid) break;
        half4 *p = reinterpret_cast<half4 *>((half_t *)ep.out + (int64_t)m * ep.ldo + n);
        half4 r = *p, o;
        for (int i = 0; i < 4; i++) o[i] = (half_t)((float)r[i] + r16(acc[i]));
        *p = o;
        break;
    }
    case EP_QKV: {
        if (!valid) break;
        const int hd = ep.hd, qrows = ep.H * hd, krows = ep.Hkv * hd;
        int b, pos;
        locate_row(m, ep.T, ep.pos_dev, ep.pos_imm, ep.pos_rows, ep.rowmap, b, pos);
        if (n < qrows + krows) {
            const int d0 = n % hd;  // multiple of 4: pairs (d0, d0+1), (d0+2, d0+3)
            const float *cs = ep.rope + ((int64_t)pos * (hd / 2) + d0 / 2) * 2;
            half4 o;
            for (int p = 0; p < 2; p++) {
                float a = r16(acc[2 * p]), bb = r16(acc[2 * p + 1]);
                float c = cs[2 * p], s = cs[2 * p + 1];
                float re = a * c - bb * s;
                float im = a * s + bb * c;
                o[2 * p] = (half_t)re;
                o[2 * p + 1] = (half_t)im;
            }
            if (n < qrows) {
                *reinterpret_cast<half4 *>((half_t *)ep.out + (int64_t)m * ep.ldo + n) = o;
            } else {
                const int kvh = (n - qrows) / hd;
                int off;
                const int64_t st = kv_stream(ep.pg, b, kvh, pos, ep.Hkv, off);
                *reinterpret_cast<half4 *>((half_t *)ep.kcache + k16_offset(st, off, d0, ep.S, hd)) = o;
            }
        } else {
            const int r = n - qrows - krows, kvh = r / hd, d0 = r % hd;
            int off;
            const int64_t st = kv_stream(ep.pg, b, kvh, pos, ep.Hkv, off);
            half_t *vc = (half_t *)ep.vcache + v16_offset(st, off, d0, ep.S, hd);
            for (int i = 0; i < 4; i++) vc[i * 32] = (half_t)acc[i];
        }
        break;
    }
    case EP_SWIGLU: {
        // packed rows 16j..16j+7 are w1 rows 8j.., rows 16j+8.. are w3 rows:
        // lanes of groups 0/1 hold a, groups 2/3 hold the matching b.
        float bv[4];
        for (int i = 0; i < 4; i++) bv[i] = __shfl_xor(acc[i], 32);
        if (!valid || g >= 2) break;
        const int f0 = (n0 >> 4) * 8 + 4 * g;
        half4 o;
        for (int i = 0; i < 4; i++) {
            float a = r16(acc[i]);
            float s = r16(a / (1.0f + expf(-a)));
            o[i] = (half_t)(s * r16(bv[i]));
        }
        half_t *gp = (half_t *)ep.out + act_offset(m, f0, ep.ldo, ep.ldo, ep.out_lay);
        *reinterpret_cast<half4 *>(gp) = o;
        break;
    }
    }
}

// ---------------------------------------------------------------------------
// Skinny product for M <= 32 rows (decode steps, short prompts): weight
// streaming.  A work-group owns TPB consecutive 16-row tiles of W and its NW
// waves interleave over K: in each round the work-group reads NW*U
// consecutive 1 KiB tiles of every owned row block (wave w the U tiles
// starting at w*U) straight into VGPRs.  The per-wave fragments are summed in
// wave order through LDS.
//
// STAGE (M <= 2): the activation rows are first copied into LDS by the whole
// work-group while the first round of weight tiles is in flight; with NORM
// they are RMS-normalised there (walkthrough section 3.2: r = 1/sqrt(mean
// x^2 + eps), round(round(x r) w)), so the normalisation costs no launch.
// Without STAGE, activation fragments are loaded from global memory (cache)
// once per round and reused for the TPB row blocks.  XT: the activations are
// fragment-major (one 1 KiB block per k-tile and 16-row half).  PF: two
// weight rounds in flight per wave (below).  NT: non-temporal weight loads
// (each weight byte is read once per step).  None of these changes the sums.
// ---------------------------------------------------------------------------
constexpr int STAGE_MAX_BYTES = 48 * 1024;

// NT: the weight stream is read with non-temporal loads
template <bool NT>
__device__ __forceinline__ half8 ldw1(const half8 *p)
{
    if (NT) return __builtin_nontemporal_load(p);
    return *p;
}

template <int NW, int U, int TPB, bool TWO, bool STAGE, bool NORM, bool XT = false, bool PF = false, bool NT = false,
          int SPL = 1>
__global__ __launch_bounds__(NW * 64) void gemm_skinny_kernel(const half_t *__restrict__ W,
                                                              const half_t *__restrict__ X,
                                                              int64_t ldx, int M, int N, int K,
                                                              Epilogue ep, const half_t *__restrict__ nw,
                                                              float eps, const int32_t *__restrict__ gtok,
                                                              int64_t gtok_ld, half_t *__restrict__ xres)
{
    extern __shared__ half8 xs[];  // STAGE: [M][K/8]
    // per-wave partial fragments of RC row blocks at a time (at most 32 KiB)
    constexpr int RC = TPB < 32 / (NW * (TWO ? 2 : 1)) ? TPB : 32 / (NW * (TWO ? 2 : 1));
    __shared__ floatx4 red[NW][RC][TWO ? 2 : 1][64];
    __shared__ float pss[NW][2];
    // SPL > 1: split K, work-group (x, y) takes k-tiles [y KT/SPL, (y+1) KT/SPL)
    // of its row blocks and stores fp32 partial sums (fragment-major X only)
    static_assert(SPL == 1 || (XT && !STAGE), "split K takes fragment-major activations");
    const int nt0 = blockIdx.x * TPB;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int KS = K >> 5, K8 = K >> 3;        // k-tiles of a W row block (its stride)
    const int KT = KS / SPL, kt0 = SPL > 1 ? blockIdx.y * KT : 0;  // this work-group's k-tiles
    const half8 *Wt = reinterpret_cast<const half8 *>(W) + ((int64_t)nt0 * KS + kt0) * 64 + lane;
    const int mc = lane & 15, g = lane >> 4;
    const bool h0 = mc < M, h1 = mc + 16 < M;
    const half8 z = {};

    int base = wave * U;
    half8 w[TPB][U];
#pragma unroll
    for (int t = 0; t < TPB; t++)
#pragma unroll
        for (int u = 0; u < U; u++)
            w[t][u] = PF ? ldw1<NT>(Wt + ((int64_t)t * KS + min(base + u, KT - 1)) * 64)
                         : (base + u < KT) ? ldw1<NT>(Wt + ((int64_t)t * KS + base + u) * 64) : z;

    if (STAGE) {
        for (int m = 0; m < M; m++) {
            // gtok: X is the embedding table and row m embeds token
            // gtok[b][pos] of its (b, pos); work-group 0 also stores the row
            // into the residual stream xres
            const half_t *xrow = X + (int64_t)m * ldx;
            if (gtok) {
                int b, pos;
                locate_row(m, ep.T, ep.pos_dev, ep.pos_imm, ep.pos_rows, ep.rowmap, b, pos);
                xrow = X + (int64_t)gtok[(int64_t)b * gtok_ld + pos] * ldx;
            }
            float ss = 0.f;
            for (int i = tid; i < K8; i += NW * 64) {
                half8 v = reinterpret_cast<const half8 *>(xrow)[i];
                xs[m * K8 + i] = v;
                if (gtok && blockIdx.x == 0) reinterpret_cast<half8 *>(xres + (int64_t)m * K)[i] = v;
                if (NORM) {
#pragma unroll
                    for (int e = 0; e < 8; e++) { float f = (float)v[e]; ss += f * f; }
                }
            }
            if (NORM) {
#pragma unroll
                for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
                if (lane == 0) pss[wave][m] = ss;
            }
        }
        __syncthreads();
        if (NORM) {
#pragma clang fp contract(off)
            for (int m = 0; m < M; m++) {
                float t = 0.f;
                for (int ww = 0; ww < NW; ww++) t += pss[ww][m];
                const float r = __frcp_rn(__fsqrt_rn(t / (float)K + eps));
                for (int i = tid; i < K8; i += NW * 64) {
                    half8 v = xs[m * K8 + i], wv = reinterpret_cast<const half8 *>(nw)[i];
#pragma unroll
                    for (int e = 0; e < 8; e++) {
                        float n = (float)(half_t)((float)v[e] * r);
                        v[e] = (half_t)(n * (float)wv[e]);
                    }
                    xs[m * K8 + i] = v;
                }
            }
            __syncthreads();
        }
    }
    const half_t *x0 = X + (int64_t)(h0 ? mc : 0) * ldx + 8 * g;
    const half_t *x1 = X + (int64_t)(h1 ? mc + 16 : 0) * ldx + 8 * g;
    const half8 *xl = STAGE ? xs + (h0 ? mc : 0) * K8 + g : nullptr;
    // fragment-major X: block (kt, half) is 64 lanes x 16 bytes
    constexpr int MH = TWO ? 2 : 1;
    const half8 *xt = reinterpret_cast<const half8 *>(X) + (int64_t)kt0 * MH * 64 + lane;

    floatx4 acc[TPB][TWO ? 2 : 1];
#pragma unroll
    for (int t = 0; t < TPB; t++)
#pragma unroll
        for (int c = 0; c < (TWO ? 2 : 1); c++) acc[t][c] = floatx4{0.f, 0.f, 0.f, 0.f};

    if (PF) {
        // Two weight rounds in flight per wave: each round issues its
        // activation loads, then the next round's weight tiles, then waits
        // only for its own operands (loads retire in issue order).  The
        // rounds of a wave are counted up front and the last one, which
        // prefetches nothing, is peeled, so the loop body has no branch and
        // the compiler's wait counts stay exact.
        constexpr int STEP = NW * U;
        const int nr = base < KT ? (KT - base + STEP - 1) / STEP : 0;
        half8 w2[TPB][U];
        auto ldw = [&](half8 (&d)[TPB][U], int b) {
#pragma unroll
            for (int t = 0; t < TPB; t++)
#pragma unroll
                for (int u = 0; u < U; u++) d[t][u] = ldw1<NT>(Wt + ((int64_t)t * KS + min(b + u, KT - 1)) * 64);
        };
        // XPF (fragment-major activations from global memory): the next
        // round's activation fragments are loaded with its weight tiles, one
        // round ahead, instead of at the start of the round that uses them
        constexpr bool XPF = XT && !STAGE;
        constexpr int U1 = TWO ? U : 1;
        half8 xa0[XPF ? U : 1], xa1[XPF ? U1 : 1], xb0[XPF ? U : 1], xb1[XPF ? U1 : 1];
        auto ldx = [&](half8 (&d0)[XPF ? U : 1], half8 (&d1)[XPF ? U1 : 1], int b) {
#pragma unroll
            for (int u = 0; u < (XPF ? U : 0); u++) {
                const int kt = min(b + u, KT - 1);
                d0[u] = xt[(int64_t)kt * MH * 64];
                if (TWO) d1[TWO ? u : 0] = xt[((int64_t)kt * MH + 1) * 64];
            }
        };
        auto round = [&](half8 (&wc)[TPB][U], half8 (&wn)[TPB][U], half8 (&xc0)[XPF ? U : 1],
                         half8 (&xc1)[XPF ? U1 : 1], half8 (&xn0)[XPF ? U : 1], half8 (&xn1)[XPF ? U1 : 1],
                         int b, bool pre) {
            half8 b0[U], b1[TWO ? U : 1];
#pragma unroll
            for (int u = 0; u < U; u++) {
                const int kt = min(b + u, KT - 1);
                if (XPF) {
                    b0[u] = xc0[XPF ? u : 0];
                    if (TWO) b1[TWO ? u : 0] = xc1[XPF && TWO ? u : 0];
                    continue;
                }
                if (STAGE) b0[u] = xl[kt * 4];
                else if (XT) b0[u] = xt[(int64_t)kt * MH * 64];
                else b0[u] = *reinterpret_cast<const half8 *>(x0 + kt * 32);
                if (TWO) {
                    if (XT) b1[TWO ? u : 0] = xt[((int64_t)kt * MH + 1) * 64];
                    else b1[TWO ? u : 0] = *reinterpret_cast<const half8 *>(x1 + kt * 32);
                }
            }
            if (pre) {
                ldw(wn, b + STEP);
                if (XPF) ldx(xn0, xn1, b + STEP);
            }
            // keep the scheduler from sinking the prefetch below the MFMAs
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < U; u++) {
                // past the end of K (last round) both operands are zero, as
                // are the rows past M
                const bool in = b + u < KT;
                const half8 a0 = (in && h0) ? b0[u] : z;
                const half8 a1 = (TWO && in && h1) ? b1[TWO ? u : 0] : z;
#pragma unroll
                for (int t = 0; t < TPB; t++) {
                    const half8 wv = in ? wc[t][u] : z;
                    acc[t][0] = mfma16(wv, a0, acc[t][0]);
                    if (TWO) acc[t][TWO ? 1 : 0] = mfma16(wv, a1, acc[t][TWO ? 1 : 0]);
                }
            }
        };
        if (XPF) ldx(xa0, xa1, base);
        int i = 0;
        for (; i + 2 < nr; i += 2) {
            round(w, w2, xa0, xa1, xb0, xb1, base, true);
            base += STEP;
            round(w2, w, xb0, xb1, xa0, xa1, base, true);
            base += STEP;
        }
        if (nr - i == 2) {
            round(w, w2, xa0, xa1, xb0, xb1, base, true);
            base += STEP;
            round(w2, w, xb0, xb1, xa0, xa1, base, false);
        } else if (nr - i == 1) {
            round(w, w2, xa0, xa1, xb0, xb1, base, false);
        }
    }
    for (; !PF && base < KT; base += NW * U) {
        half8 b0[U], b1[TWO ? U : 1];
#pragma unroll
        for (int u = 0; u < U; u++) {
            const bool ok = h0 && base + u < KT;
            if (STAGE) b0[u] = ok ? xl[(base + u) * 4] : z;
            else if (XT) b0[u] = ok ? xt[(int64_t)(base + u) * MH * 64] : z;
            else b0[u] = ok ? *reinterpret_cast<const half8 *>(x0 + (base + u) * 32) : z;
        }
        if (TWO) {
#pragma unroll
            for (int u = 0; u < U; u++) {
                const bool ok = h1 && base + u < KT;
                if (XT) b1[u] = ok ? xt[((int64_t)(base + u) * MH + 1) * 64] : z;
                else b1[u] = ok ? *reinterpret_cast<const half8 *>(x1 + (base + u) * 32) : z;
            }
        }
#pragma unroll
        for (int t = 0; t < TPB; t++)
#pragma unroll
            for (int u = 0; u < U; u++) {
                acc[t][0] = mfma16(w[t][u], b0[u], acc[t][0]);
                if (TWO) acc[t][TWO ? 1 : 0] = mfma16(w[t][u], b1[TWO ? u : 0], acc[t][TWO ? 1 : 0]);
            }
        const int nb = base + NW * U;
        if (nb < KT) {
#pragma unroll
            for (int t = 0; t < TPB; t++)
#pragma unroll
                for (int u = 0; u < U; u++) w[t][u] = (nb + u < KT) ? ldw1<NT>(Wt + ((int64_t)t * KS + nb + u) * 64) : z;
        }
    }
    // the waves' fragments are summed in wave order, RC row blocks at a
    // time; one accumulator fragment (row block t, row half c) per wave
    constexpr int C = TWO ? 2 : 1;
#pragma unroll
    for (int t0 = 0; t0 < TPB; t0 += RC) {
        if (t0) __syncthreads();  // the previous chunk has been read
#pragma unroll
        for (int t = 0; t < RC; t++)
#pragma unroll
            for (int c = 0; c < C; c++)
                if (t0 + t < TPB) red[wave][t][c][lane] = acc[t0 + t < TPB ? t0 + t : 0][c];
        __syncthreads();
        for (int pi = wave; pi < RC * C; pi += NW) {
            const int t = pi / C, c = pi % C;
            if (t0 + t >= TPB) continue;
            floatx4 s0 = red[0][t][c][lane];
            for (int ww = 1; ww < NW; ww++) s0 += red[ww][t][c][lane];
            if (SPL > 1) {
                const int m = mc + 16 * c;
                if (c ? h1 : h0)
                    *reinterpret_cast<floatx4 *>(ep.part + ((int64_t)blockIdx.y * M + m) * N + (nt0 + t0 + t) * 16 +
                                                 4 * g) = s0;
            } else {
                epilogue_frag(ep, (nt0 + t0 + t) * 16, mc + 16 * c, c ? h1 : h0, s0, lane);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Tiled product for M > 32 (prefill).  Block tile 128 (W rows) x 128 (tokens)
// x 64 (K), four waves in a 2x2 arrangement, each owning 4x4 fragments.
// W tiles are copied to LDS unchanged (their lane order is the operand
// order); X rows are scattered into the same lane order.  Double-buffered
// LDS with register prefetch of the next K slab.  Work-groups are remapped
// so that the ones on one XCD (dispatch is round-robin over 8) take adjacent
// tiles, and grouped GM token blocks at a time so W slabs are reused from
// cache.
// ---------------------------------------------------------------------------
constexpr int BIG_BN = 128, BIG_BM = 128, BIG_GM = 8;

__global__ __launch_bounds__(256) void gemm_big_kernel(const half_t *__restrict__ W,
                                                       const half_t *__restrict__ X, int64_t ldx,
                                                       int M, int N, int K, Epilogue ep)
{
    __shared__ half8 lw[2][16 * 64];
    __shared__ half8 lx[2][16 * 64];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wn = wave >> 1, wm = wave & 1;
    const int NB = (N + BIG_BN - 1) / BIG_BN, MB = (M + BIG_BM - 1) / BIG_BM;
    const int total = NB * MB;

    // XCD-aware remap of the dispatch index.
    int pid = blockIdx.x;
    {
        int per = total / 8, rem = total % 8, xcd = pid % 8, local = pid / 8;
        pid = xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
    }
    const int group = BIG_GM * NB;
    const int first_mb = (pid / group) * BIG_GM;
    const int gm = min(MB - first_mb, BIG_GM);
    const int mb = first_mb + (pid % group) % gm;
    const int nb = (pid % group) / gm;

    const int KT = K >> 5, NT = N >> 4;
    const half8 *Wv = reinterpret_cast<const half8 *>(W);
    const half8 z = {};

    half8 rw[4], rx[4];
    auto load_slab = [&](int kb) {
#pragma unroll
        for (int j = 0; j < 4; j++) {
            int c = tid + 256 * j;
            int ntl = c >> 7, within = c & 127;
            int ntg = nb * 8 + ntl;
            rw[j] = ntg < NT ? Wv[((int64_t)ntg * KT + kb * 2) * 64 + within] : z;
            int m = c >> 3, ch = c & 7;
            int mg = mb * BIG_BM + m;
            rx[j] = mg < M ? *reinterpret_cast<const half8 *>(X + (int64_t)mg * ldx + kb * 64 + ch * 8) : z;
        }
    };
    auto store_slab = [&](int buf) {
#pragma unroll
        for (int j = 0; j < 4; j++) {
            int c = tid + 256 * j;
            lw[buf][c] = rw[j];
            int m = c >> 3, ch = c & 7;
            int mt = m >> 4, kt = ch >> 2, ln = (m & 15) + 16 * (ch & 3);
            lx[buf][(mt * 2 + kt) * 64 + ln] = rx[j];
        }
    };

    floatx4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    const int nkb = K / 64;
    load_slab(0);
    store_slab(0);
    __syncthreads();
    for (int kb = 0; kb < nkb; kb++) {
        const int cur = kb & 1;
        if (kb + 1 < nkb) load_slab(kb + 1);
#pragma unroll
        for (int kt = 0; kt < 2; kt++) {
            half8 a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; i++) a[i] = lw[cur][((wn * 4 + i) * 2 + kt) * 64 + lane];
#pragma unroll
            for (int j = 0; j < 4; j++) b[j] = lx[cur][((wm * 4 + j) * 2 + kt) * 64 + lane];
#pragma unroll
            for (int i = 0; i < 4; i++)
#pragma unroll
                for (int j = 0; j < 4; j++) acc[i][j] = mfma16(a[i], b[j], acc[i][j]);
        }
        if (kb + 1 < nkb) store_slab(cur ^ 1);
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int n0 = (nb * 8 + wn * 4 + i) * 16;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int m = (mb * 8 + wm * 4 + j) * 16 + (lane & 15);
            epilogue_frag(ep, n0, m, m < M && n0 < N, acc[i][j], lane);
        }
    }
}

// ---------------------------------------------------------------------------
// Large prefill product (M >= 1024): block tile 256 (W rows) x 256 (tokens) x
// 32 (K) per work-group, eight waves in a 2 x 4 arrangement each owning
// 128 x 64 (32 accumulator fragments), two waves per SIMD.  Operands travel
// global -> LDS with direct loads (global_load_lds_dwordx4): each wave copies
// two 1 KiB W tiles (the stored layout is already the operand order) and two
// X tiles, through a ring of NS stages so that NS-2 stages of loads stay in
// flight while one is multiplied.  Waits are explicit counter waits plus a
// bare s_barrier (a full __syncthreads would drain the in-flight stages every
// step).  Each wave reads its 12 operand fragments of a k-tile before its 32
// MFMAs (a scheduling barrier keeps the reads together) and starts each
// column group as soon as its fragment is in.  Rows past N or M are clamped
// on load (never stored).  XT: X is stored in the weight tile layout
// (ACT_TILED), so its copies are as contiguous as the weights'; otherwise X
// is row-major with stride ldx.  (Products with X in the tile layout are
// launched in the register form below; this kernel takes row-major X.)
// ---------------------------------------------------------------------------

template <int NS>
__device__ __forceinline__ void wait_vm_in_flight8(bool keep)
{
    // keep: the NS-2 newest stages (4 loads each per wave) stay in flight
    static_assert(NS == 4 || NS == 5, "four or five stages");
    if (!keep) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    else if (NS == 4) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
}

template <bool XT, int KIND, int NS = 4>
__global__ __launch_bounds__(512, 1) void gemm_tile256_kernel(const half_t *__restrict__ W,
                                                                 const half_t *__restrict__ X, int64_t ldx,
                                                                 int M, int N, int K, Epilogue ep)
{
    extern __shared__ half8 lds[];
    half8 *lw = lds;              // [NS][16 tiles][64 lanes]
    half8 *lx = lds + NS * 1024;  // [NS][16 tiles][64 lanes]
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int wn = wave >> 2, wm = wave & 3;
    const int NB = (N + 255) / 256, MB = (M + 255) / 256;
    const int total = NB * MB;
    int pid = blockIdx.x;
    {  // XCD-aware remap, then groups of 4 token blocks per W block column
        int per = total / 8, rem = total % 8, xcd = pid % 8, local = pid / 8;
        pid = xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
    }
    const int group = 4 * NB;
    const int first_mb = (pid / group) * 4;
    const int gm = min(MB - first_mb, 4);
    const int mb = first_mb + (pid % group) % gm;
    const int nb = (pid % group) / gm;

    const int KT = K >> 5, NT = N >> 4, MT = (M + 15) >> 4;
    const half8 *Wv = reinterpret_cast<const half8 *>(W);
    const half8 *wsrc[2];
    const half_t *xsrc[2];
#pragma unroll
    for (int q = 0; q < 2; q++) {
        const int tile = wave * 2 + q;
        wsrc[q] = Wv + (int64_t)min(nb * 16 + tile, NT - 1) * KT * 64 + lane;
        if (XT) {
            xsrc[q] = X + ((int64_t)min(mb * 16 + tile, MT - 1) * KT * 64 + lane) * 8;
        } else {
            const int m = min(mb * 256 + tile * 16 + (lane & 15), M - 1);
            xsrc[q] = X + (int64_t)m * ldx + 8 * (lane >> 4);
        }
    }
    auto issue = [&](int st) {
        const int buf = st % NS;
#pragma unroll
        for (int q = 0; q < 2; q++) {
            const int tile = wave * 2 + q;
            lds_copy16(wsrc[q] + (int64_t)st * 64, lw + buf * 1024 + tile * 64);
            lds_copy16(xsrc[q] + (XT ? (int64_t)st * 512 : (int64_t)st * 32), lx + buf * 1024 + tile * 64);
        }
    };
    floatx4 acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int st = 0; st < NS - 1; st++)
        if (st < KT) issue(st);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the epilogue's scalar argument loads
    for (int kt = 0; kt < KT; kt++) {
        wait_vm_in_flight8<NS>(kt + NS - 2 < KT);
        __builtin_amdgcn_s_barrier();
        const int nk = kt + NS - 1;
        if (nk < KT) issue(nk);
        const int cur = kt % NS;
        half8 a[8], b[4];
#pragma unroll
        for (int i = 0; i < 8; i++) a[i] = lw[cur * 1024 + (wn * 8 + i) * 64 + lane];
#pragma unroll
        for (int j = 0; j < 4; j++) b[j] = lx[cur * 1024 + (wm * 4 + j) * 64 + lane];
        __builtin_amdgcn_sched_barrier(0);
        // raised wave priority while this wave has MFMAs to issue, so the
        // SIMD's other wave (waiting on LDS or the barrier) does not take
        // its issue slots (measured 2-7% on the prefill shapes)
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int j = 0; j < 4; j++) {
            switch (j) {
            case 0: asm volatile("s_waitcnt lgkmcnt(3)" ::: "memory"); break;
            case 1: asm volatile("s_waitcnt lgkmcnt(2)" ::: "memory"); break;
            case 2: asm volatile("s_waitcnt lgkmcnt(1)" ::: "memory"); break;
            default: asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); break;
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < 8; i++) acc[i][j] = mfma16(a[i], b[j], acc[i][j]);
            __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_setprio(0);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const int n0 = (nb * 16 + wn * 8 + i) * 16;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int m = (mb * 16 + wm * 4 + j) * 16 + (lane & 15);
            epilogue_frag<KIND>(ep, n0, m, m < M && n0 < N, acc[i][j], lane);
        }
    }
}

// ---------------------------------------------------------------------------
// The same product when X is stored in the weight tile layout (ACT_TILED):
// each wave loads its four X fragments of a k-tile straight from global
// memory into registers, two k-tiles ahead, and only W goes through the LDS
// ring (NSW stages of 16 KiB), whose fragments for the next k-tile are read
// while the current one multiplies.  A third fewer LDS reads and half the
// LDS copies; measured 4-7% faster than the form above on the 7B..70B
// prefill shapes (interleaved runs, medians), with the same sums.  Every wave
// issues per k-tile its two W copies and its X loads unconditionally
// (indexes past the end are clamped and the results never used) and in a
// fixed order, so that counter waits cover both operands.
// ---------------------------------------------------------------------------
// s_waitcnt vmcnt(0) with the other counters left alone (gfx9 encoding)
constexpr int kVmcnt0 = 0x0F70;

// The epilogue of one wave's share of a tile: 8 x XF accumulator fragments,
// fragment (i, j) holding W rows nrow0 + 16 i .. +15 (of this launch, whose
// first row is n_base) and tokens mtok0 + 16 j .. +15, with the arithmetic
// of epilogue_frag element for element.  The memory a kind reads (the
// residual rows, the rotation table, the row positions) is loaded for a
// group of fragments before any of their results is stored, so a wave waits
// on memory once per group instead of once per fragment.  SWIGLU swaps the
// halves of each (a, b) fragment pair between lanes 32 apart (which hold a
// and b of the same outputs), so every lane computes two outputs instead of
// half the lanes computing four.
template <int KIND, int XF>
__device__ __forceinline__ void epilogue_tile(const Epilogue &ep, floatx4 (&acc)[8][XF], int nrow0, int mtok0,
                                              int M, int N, int n_base, int lane)
{
#pragma clang fp contract(off)
    const int g = lane >> 4;
    if constexpr (KIND == EP_RESID) {
        half4 rv[8][XF];
#pragma unroll
        for (int i = 0; i < 8; i++)
#pragma unroll
            for (int j = 0; j < XF; j++) {
                const int n0 = nrow0 + 16 * i, m = mtok0 + 16 * j + (lane & 15);
                rv[i][j] = half4{};
                if (m < M && n0 < N)
                    rv[i][j] = *reinterpret_cast<const half4 *>((const half_t *)ep.out + (int64_t)m * ep.ldo + n_base +
                                                                n0 + 4 * g);
            }
        // one wait for all of them, outside the per-fragment branches (which
        // the compiler would otherwise give a wait each)
        __builtin_amdgcn_s_waitcnt(kVmcnt0);
#pragma unroll
        for (int i = 0; i < 8; i++)
#pragma unroll
            for (int j = 0; j < XF; j++) {
                const int n0 = nrow0 + 16 * i, m = mtok0 + 16 * j + (lane & 15);
                if (!(m < M && n0 < N)) continue;
                half4 o;
                for (int e = 0; e < 4; e++) o[e] = (half_t)((float)rv[i][j][e] + r16(acc[i][j][e]));
                *reinterpret_cast<half4 *>((half_t *)ep.out + (int64_t)m * ep.ldo + n_base + n0 + 4 * g) = o;
            }
    } else if constexpr (KIND == EP_SWIGLU) {
        const int hi = g >> 1;  // lanes 32..63: outputs 2 and 3 of the group
#pragma unroll
        for (int i = 0; i < 8; i++)
#pragma unroll
            for (int j = 0; j < XF; j++) {
                const int n0 = nrow0 + 16 * i, m = mtok0 + 16 * j + (lane & 15);
                // lanes 0..31 hold a (w1 rows), lanes 32..63 the matching b
                // (w3 rows); after the swaps s[k][0] is a and s[k][1] is b of
                // this lane's output k (outputs 0, 1 below lane 32, 2, 3 above)
                const auto s0 = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[i][j][0]),
                                                                 __float_as_uint(acc[i][j][2]), false, false);
                const auto s1 = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[i][j][1]),
                                                                 __float_as_uint(acc[i][j][3]), false, false);
                if (!(m < M && n0 < N)) continue;
                const float av[2] = {__uint_as_float(s0[0]), __uint_as_float(s1[0])};
                const float bv[2] = {__uint_as_float(s0[1]), __uint_as_float(s1[1])};
                half2v o;
                for (int k = 0; k < 2; k++) {
                    const float a = r16(av[k]);
                    const float sl = r16(a / (1.0f + expf(-a)));
                    o[k] = (half_t)(sl * r16(bv[k]));
                }
                const int f0 = ((n_base + n0) >> 4) * 8 + 4 * (g & 1);
                *reinterpret_cast<half2v *>((half_t *)ep.out + act_offset(m, f0, ep.ldo, ep.ldo, ep.out_lay) + 2 * hi) = o;
            }
    } else if constexpr (KIND == EP_QKV) {
        // head dimension 128 (checked by the launcher): the divisions below
        // are shifts
        constexpr int hd = 128;
        const int qrows = ep.H * hd, krows = ep.Hkv * hd;
        int bj[XF], pj[XF];
#pragma unroll
        for (int j = 0; j < XF; j++) {
            const int m = mtok0 + 16 * j + (lane & 15);
            bj[j] = pj[j] = 0;
            if (m < M) locate_row(m, ep.T, ep.pos_dev, ep.pos_imm, ep.pos_rows, ep.rowmap, bj[j], pj[j]);
        }
        __builtin_amdgcn_s_waitcnt(kVmcnt0);
#pragma unroll
        for (int i0 = 0; i0 < 8; i0 += 4) {
            float4 cs[4][XF];
#pragma unroll
            for (int i = 0; i < 4; i++)
#pragma unroll
                for (int j = 0; j < XF; j++) {
                    const int n0 = n_base + nrow0 + 16 * (i0 + i), n = n0 + 4 * g;
                    const int m = mtok0 + 16 * j + (lane & 15);
                    cs[i][j] = make_float4(0.f, 0.f, 0.f, 0.f);
                    if (m < M && n0 - n_base < N && n < qrows + krows)
                        cs[i][j] = *reinterpret_cast<const float4 *>(ep.rope + ((int64_t)pj[j] * (hd / 2) + n % hd / 2) * 2);
                }
            __builtin_amdgcn_s_waitcnt(kVmcnt0);
#pragma unroll
            for (int i = 0; i < 4; i++)
#pragma unroll
                for (int j = 0; j < XF; j++) {
                    const int n0 = n_base + nrow0 + 16 * (i0 + i), n = n0 + 4 * g;
                    const int m = mtok0 + 16 * j + (lane & 15);
                    if (!(m < M && n0 - n_base < N)) continue;
                    const floatx4 &ac = acc[i0 + i][j];
                    if (n < qrows + krows) {
                        const int d0 = n % hd;  // multiple of 4: pairs (d0, d0+1), (d0+2, d0+3)
                        const float c4[4] = {cs[i][j].x, cs[i][j].y, cs[i][j].z, cs[i][j].w};
                        half4 o;
                        for (int q = 0; q < 2; q++) {
                            const float a = r16(ac[2 * q]), bb = r16(ac[2 * q + 1]);
                            const float c = c4[2 * q], sn = c4[2 * q + 1];
                            const float re = a * c - bb * sn;
                            const float im = a * sn + bb * c;
                            o[2 * q] = (half_t)re;
                            o[2 * q + 1] = (half_t)im;
                        }
                        if (n < qrows) {
                            *reinterpret_cast<half4 *>((half_t *)ep.out + (int64_t)m * ep.ldo + n) = o;
                        } else {
                            const int kvh = (n - qrows) / hd;
                            int off;
                            const int64_t st = kv_stream(ep.pg, bj[j], kvh, pj[j], ep.Hkv, off);
                            *reinterpret_cast<half4 *>((half_t *)ep.kcache + k16_offset(st, off, d0, ep.S, hd)) = o;
                        }
                    } else {
                        const int r = n - qrows - krows, kvh = r / hd, d0 = r % hd;
                        int off;
                        const int64_t st = kv_stream(ep.pg, bj[j], kvh, pj[j], ep.Hkv, off);
                        half_t *vc = (half_t *)ep.vcache + v16_offset(st, off, d0, ep.S, hd);
                        for (int e = 0; e < 4; e++) vc[e * 32] = (half_t)ac[e];
                    }
                }
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; i++)
#pragma unroll
            for (int j = 0; j < XF; j++) {
                const int n0 = nrow0 + 16 * i, m = mtok0 + 16 * j + (lane & 15);
                epilogue_frag<KIND>(ep, n_base + n0, m, m < M && n0 < N, acc[i][j], lane);
            }
    }
}

template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int KIND, int NSW, int PD, int TOK = 256>
__global__ __launch_bounds__(512, 1) void gemm_tile256_xreg_kernel(const half_t *__restrict__ W, const half_t *X,
                                                                      int M, int N, int K, int n_base, Epilogue ep)
{
    static_assert(PD == 2 && NSW == 5, "the counter waits below are for this ring and two k-tiles of X in flight");
    static_assert(TOK == 256 || TOK == 128, "token tiles of 256 or 128");
    constexpr int XF = TOK / 64;  // X fragments per wave and k-tile
    extern __shared__ half8 lds[];
    half8 *lw = lds;  // [NSW][16 tiles][64 lanes]
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int wn = wave >> 2, wm = wave & 3;
    const int NB = (N + 255) / 256, MB = (M + TOK - 1) / TOK;
    const int total = NB * MB;
    int pid = blockIdx.x;
    {  // XCD-aware remap, then groups of 4 token blocks per W block column
        int per = total / 8, rem = total % 8, xcd = pid % 8, local = pid / 8;
        pid = xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
    }
    const int group = 4 * NB;
    const int first_mb = (pid / group) * 4;
    const int gm = min(MB - first_mb, 4);
    const int mb = first_mb + (pid % group) % gm;
    const int nb = (pid % group) / gm;

    const int KT = K >> 5, NT = N >> 4, MT = (M + 15) >> 4;
    const half8 *Wv = reinterpret_cast<const half8 *>(W), *Xv = reinterpret_cast<const half8 *>(X);
    const half8 *wsrc[2], *xsrc[XF];
#pragma unroll
    for (int q = 0; q < 2; q++) wsrc[q] = Wv + (int64_t)min(nb * 16 + wave * 2 + q, NT - 1) * KT * 64 + lane;
#pragma unroll
    for (int j = 0; j < XF; j++) xsrc[j] = Xv + (int64_t)min(mb * (TOK / 16) + wm * XF + j, MT - 1) * KT * 64 + lane;
    auto issue_w = [&](int st) {  // stage st into buffer st % NSW; past the end: never read
        const int buf = st % NSW, k = min(st, KT - 1);
#pragma unroll
        for (int q = 0; q < 2; q++) lds_copy16(wsrc[q] + (int64_t)k * 64, lw + buf * 1024 + (wave * 2 + q) * 64);
    };
    half8 xb[PD][XF];
    auto copy_w1 = [&](int st, int q) {
        lds_copy16(wsrc[q] + (int64_t)min(st, KT - 1) * 64, lw + (st % NSW) * 1024 + (wave * 2 + q) * 64);
    };
    // one X fragment of k-tile kt into d, from assembly like the copies, so
    // that the compiler adds no waits of its own: the counter waits below
    // cover both (indexes past the end are clamped, the results unused)
    auto load_x1 = [&](int kt, int j, half8 &d) {
        asm volatile("global_load_dwordx4 %0, %1, off"
                     : "=v"(d)
                     : "v"(xsrc[j] + (int64_t)min(kt, KT - 1) * 64)
                     : "memory");
    };
    floatx4 acc[8][XF];
#pragma unroll
    for (int i = 0; i < 8; i++)
#pragma unroll
        for (int j = 0; j < XF; j++) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    // W stages 0..NSW-2-PD alone, then PD (W, X) groups as the loop issues them
    for (int st = 0; st <= NSW - 2 - PD; st++) issue_w(st);
#pragma unroll
    for (int p = 0; p < PD; p++) {
        issue_w(NSW - 1 - PD + p);
#pragma unroll
        for (int j = 0; j < XF; j++)
            if (p == 0 || j < XF - 1) load_x1(p, j, xb[p][j]);
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the epilogue's scalar argument loads
    // The A fragments of k-tile kt+1 are read from LDS while k-tile kt
    // multiplies (two register sets, alternating with the unrolled body).
    // Stage 0 first: after its copies this wave has issued W(1), W(2), X(0),
    // W(3) and X(1) but its last fragment (which k-tile 0 loads), i.e.
    // 6 + 2 XF - 1 operations.
    wait_vmcnt<3 * 2 + 2 * XF - 1>();
    __builtin_amdgcn_s_barrier();
    half8 ab[PD][8];
#pragma unroll
    for (int i = 0; i < 8; i++) ab[0][i] = lw[(wn * 8 + i) * 64 + lane];
    // KT % PD == 0 (checked by the launcher): no guard inside the unrolled
    // body.  Each k-tile's copies, fragment reads and X loads are spread over
    // its MFMA groups (one per X fragment), so that neither wave of a SIMD
    // issues them in one burst.  Per k-tile, in issue order: group 0 loads
    // the last fragment of X(kt+1) after its MFMAs (into the register the
    // previous k-tile's last group read); group j > 0 issues its W copies
    // before its MFMAs and X(kt+2) fragment j-1 after them (into the register
    // group j-1 read).  A fragment register is thus reloaded at least one
    // MFMA group after its last reader, and an LDS fragment read never
    // follows an MFMA that reads the register it fills: an LDS read placed
    // directly after such an MFMA gave wrong sums (the MFMA had not yet read
    // its operand).  Counts per k-tile: CW = 2 copies, XF loads.
    constexpr int C0 = 2 / XF;                            // copies of group 0
    constexpr int TOPW = 2 + XF;                          // k-tile kt-1's operations
    constexpr int LASTW = 2 * (2 + XF - 1) - C0;          // after X(kt)'s last fragment
    for (int kt0 = 0; kt0 < KT; kt0 += PD) {
#pragma unroll
        for (int p = 0; p < PD; p++) {
            const int kt = kt0 + p;
            {
                // every operation k-tile kt-2 issued is in (k-tile kt-1's may
                // be pending): X(kt) but its last fragment, and W stages up
                // to kt+1; also the fragment reads of A(kt).  The barrier makes
                // every wave's W copies visible and tells this wave that all
                // have finished reading buffer (kt - 1) % NSW
                wait_vmcnt<TOPW>();
                __builtin_amdgcn_s_waitcnt(0xC07F);
                __builtin_amdgcn_s_barrier();
                const int nx = (kt + 1) % NSW;  // after the last k-tile: a stage never used
                // (no raised wave priority here: with the work spread over the
                // groups, either wave of a SIMD may issue; priority around the
                // MFMAs, which paid with the work in bursts, cost 1.6%)
#pragma unroll
                for (int j = 0; j < XF; j++) {
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int i = j * 8 / XF; i < (j + 1) * 8 / XF; i++)
                        ab[1 - p][i] = lw[nx * 1024 + (wn * 8 + i) * 64 + lane];
#pragma unroll
                    for (int q = j * 2 / XF; q < (j + 1) * 2 / XF; q++) copy_w1(kt + NSW - 1, q);
                    // the last group also needs X(kt)'s last fragment
                    if (j == XF - 1) wait_vmcnt<LASTW>();
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int i = 0; i < 8; i++) acc[i][j] = mfma16(ab[p][i], xb[p][j], acc[i][j]);
                    __builtin_amdgcn_sched_barrier(0);
                    if (j == 0) load_x1(kt + 1, XF - 1, xb[1 - p][XF - 1]);
                    else load_x1(kt + PD, j - 1, xb[p][j - 1]);
                }
            }
        }
    }
    // The last k-tiles' X loads are still landing in their registers, which
    // hold no value the compiler still needs: each is tied to a statement
    // after the wait, so that nothing else is put there before they land.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
    for (int p = 0; p < PD; p++)
#pragma unroll
        for (int j = 0; j < XF; j++) asm volatile("" ::"v"(xb[p][j]));
    epilogue_tile<KIND, XF>(ep, acc, (nb * 16 + wn * 8) * 16, (mb * (TOK / 16) + wm * XF) * 16, M, N, n_base, lane);
}

// One launch over W rows [n_base, n_base + N) (a whole number of 256-row
// blocks from the start of W, or the rest of it).
template <int NSW, int TOK>
hipError_t launch_xreg_part(const GemmArgs &a, int n_base, int N, hipStream_t s)
{
    constexpr int PD = 2;
    const int NB = (N + 255) / 256, MB = (a.M + TOK - 1) / TOK;
    const dim3 grid(NB * MB), blk(512);
    const size_t lds = (size_t)NSW * 1024 * 16;
    const half_t *W = (const half_t *)a.W + (int64_t)n_base * a.K, *X = (const half_t *)a.X;
    switch (a.ep.kind) {
    case EP_STORE:
        hipLaunchKernelGGL((gemm_tile256_xreg_kernel<EP_STORE, NSW, PD, TOK>), grid, blk, lds, s, W, X, a.M, N, a.K,
                           n_base, a.ep);
        break;
    case EP_RESID:
        hipLaunchKernelGGL((gemm_tile256_xreg_kernel<EP_RESID, NSW, PD, TOK>), grid, blk, lds, s, W, X, a.M, N, a.K,
                           n_base, a.ep);
        break;
    case EP_LOGITS:
        hipLaunchKernelGGL((gemm_tile256_xreg_kernel<EP_LOGITS, NSW, PD, TOK>), grid, blk, lds, s, W, X, a.M, N, a.K,
                           n_base, a.ep);
        break;
    case EP_QKV:
        hipLaunchKernelGGL((gemm_tile256_xreg_kernel<EP_QKV, NSW, PD, TOK>), grid, blk, lds, s, W, X, a.M, N, a.K,
                           n_base, a.ep);
        break;
    case EP_SWIGLU:
        hipLaunchKernelGGL((gemm_tile256_xreg_kernel<EP_SWIGLU, NSW, PD, TOK>), grid, blk, lds, s, W, X, a.M, N, a.K,
                           n_base, a.ep);
        break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// 256 x 256 tiles, one per CU at a time, so a product takes as many tile
// times as it has waves of 256 tiles.  When the last wave is at most half
// full and made of whole W block columns (rem = tiles % 256 a multiple of the
// token blocks), those columns go to a second launch of 256 x 128 tiles,
// which fills one wave with twice as many half-size tiles.  Every output is
// summed over K in the same order either way.
template <int NSW>
hipError_t launch_tile256_xreg(const GemmArgs &a, hipStream_t s)
{
    const int NB = (a.N + 255) / 256, MB = (a.M + 255) / 256;
    const int rem = (NB * MB) % 256;
    const int ncols = rem && rem <= 128 && rem % MB == 0 ? rem / MB : 0;
    if (ncols == 0 || ncols >= NB) return launch_xreg_part<NSW, 256>(a, 0, a.N, s);
    const int NA = (NB - ncols) * 256;
    const hipError_t e = launch_xreg_part<NSW, 256>(a, 0, NA, s);
    if (e != hipSuccess) return e;
    return launch_xreg_part<NSW, 128>(a, NA, a.N - NA, s);
}

template <bool XT>
hipError_t launch_tile256(const GemmArgs &a, hipStream_t s)
{
    if constexpr (XT) {
        // fp16 models have dim and ffn width multiples of 64: K/32 is even;
        // the QKV epilogue of this form takes heads of 128
        if ((a.K >> 5) % 2 || (a.ep.kind == EP_QKV && a.ep.hd != 128)) return hipErrorInvalidValue;
        return launch_tile256_xreg<5>(a, s);
    } else {
        // the eight-wave form with a five-stage ring (measured 4-16% faster than
        // four waves and four stages on the 7B..70B prefill shapes, same sums)
        constexpr int NS = 5;
        const int NB = (a.N + 255) / 256, MB = (a.M + 255) / 256;
        const dim3 grid(NB * MB), blk(512);
        const size_t lds = (size_t)NS * 2 * 1024 * 16;
        const half_t *W = (const half_t *)a.W, *X = (const half_t *)a.X;
        const int64_t ldx = XT ? 0 : a.ldx;
        switch (a.ep.kind) {
        case EP_STORE:
            hipLaunchKernelGGL((gemm_tile256_kernel<XT, EP_STORE, NS>), grid, blk, lds, s, W, X, ldx, a.M, a.N, a.K, a.ep);
            break;
        case EP_RESID:
            hipLaunchKernelGGL((gemm_tile256_kernel<XT, EP_RESID, NS>), grid, blk, lds, s, W, X, ldx, a.M, a.N, a.K, a.ep);
            break;
        case EP_LOGITS:
            hipLaunchKernelGGL((gemm_tile256_kernel<XT, EP_LOGITS, NS>), grid, blk, lds, s, W, X, ldx, a.M, a.N, a.K, a.ep);
            break;
        case EP_QKV:
            hipLaunchKernelGGL((gemm_tile256_kernel<XT, EP_QKV, NS>), grid, blk, lds, s, W, X, ldx, a.M, a.N, a.K, a.ep);
            break;
        case EP_SWIGLU:
            hipLaunchKernelGGL((gemm_tile256_kernel<XT, EP_SWIGLU, NS>), grid, blk, lds, s, W, X, ldx, a.M, a.N, a.K, a.ep);
            break;
        default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
}

// ---------------------------------------------------------------------------
// fp32 models: plain row-major weights, one thread per output unit (a row, a
// RoPE pair, or a w1/w3 pair), fp32 accumulation in k order.
// ---------------------------------------------------------------------------
__device__ float dot_row_f32(const float *w, const float *x, int K)
{
    float s = 0.f;
    for (int k = 0; k < K; k++) s = fmaf(w[k], x[k], s);
    return s;
}

__global__ void linear_f32_kernel(const float *W, const float *X, int64_t ldx, int M, int N, int K,
                                  Epilogue ep)
{
#pragma clang fp contract(off)
    const int unit = blockIdx.x * blockDim.x + threadIdx.x;
    const int m = blockIdx.y;
    const float *x = X + (int64_t)m * ldx;
    float *out = (float *)ep.out;
    switch (ep.kind) {
    case EP_STORE:
    case EP_LOGITS:
    case EP_RESID: {
        if (ep.kind == EP_LOGITS && ep.pos_advance && unit == 0 && m == 0) *ep.pos_advance += 1;
        if (unit >= N) return;
        float a = dot_row_f32(W + (int64_t)unit * K, x, K);
        float *o = out + (int64_t)m * ep.ldo + unit;
        *o = ep.kind == EP_RESID ? *o + a : a;
        break;
    }
    case EP_QKV: {
        const int n = 2 * unit;
        if (n >= N) return;
        const int hd = ep.hd, qrows = ep.H * hd, krows = ep.Hkv * hd;
        int b, pos;
        locate_row(m, ep.T, ep.pos_dev, ep.pos_imm, ep.pos_rows, ep.rowmap, b, pos);
        float a = dot_row_f32(W + (int64_t)n * K, x, K);
        float bb = dot_row_f32(W + (int64_t)(n + 1) * K, x, K);
        if (n < qrows + krows) {
            const int d0 = n % hd;
            const float *cs = ep.rope + ((int64_t)pos * (hd / 2) + d0 / 2) * 2;
            float re = a * cs[0] - bb * cs[1];
            float im = a * cs[1] + bb * cs[0];
            if (n < qrows) {
                out[(int64_t)m * ep.ldo + n] = re;
                out[(int64_t)m * ep.ldo + n + 1] = im;
            } else {
                int off;
                const int64_t st = kv_stream(ep.pg, b, (n - qrows) / hd, pos, ep.Hkv, off);
                float *kc = (float *)ep.kcache + k_offset(st, off, d0, ep.S, hd);
                kc[0] = re;
                kc[1] = im;
            }
        } else {
            const int r = n - qrows - krows, kvh = r / hd, d0 = r % hd;
            int off;
            const int64_t st = kv_stream(ep.pg, b, kvh, pos, ep.Hkv, off);
            float *vc = (float *)ep.vcache + v32_offset(st, off, d0, ep.S, hd);
            vc[0] = a;
            vc[ep.S] = bb;
        }
        break;
    }
    case EP_SWIGLU: {
        const int f = unit;
        if (f >= N / 2) return;
        const int ra = (f >> 3) * 16 + (f & 7);
        float a = dot_row_f32(W + (int64_t)ra * K, x, K);
        float b = dot_row_f32(W + (int64_t)(ra + 8) * K, x, K);
        out[(int64_t)m * ep.ldo + f] = (a / (1.0f + expf(-a))) * b;
        break;
    }
    }
}

}  // namespace

bool skinny_can_normalise(int M, int K) { return M <= 2 && (int64_t)M * K * 2 <= STAGE_MAX_BYTES; }

namespace {
// The partial sums of a split-K product added in split order, then the
// epilogue: one thread per four consecutive outputs of a row.
template <int KIND>
__global__ __launch_bounds__(256) void split_reduce_kernel(int S, int M, int N, Epilogue ep)
{
    const int n4 = N / 4;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)M * n4) return;
    const int m = (int)(i / n4), n = (int)(i % n4) * 4;
    const floatx4 *p = reinterpret_cast<const floatx4 *>(ep.part + (int64_t)m * N + n);
    const int64_t stride = (int64_t)M * n4;
    floatx4 sum = p[0];
    for (int s = 1; s < S; s++) sum += p[s * stride];
    epilogue_frag<KIND>(ep, n, m, true, sum, 0);
}
}  // namespace

// Fragment-major rows (TWO: 17..32, else up to 16): SPL work-groups share
// each group of TPB row blocks, each over 1/SPL of K, then one reduce launch
// applies the epilogue (kinds that work on four outputs of a row at a time:
// store, residual, qkv)
template <int U, int TPB, bool PF, int SPL, bool TWO = true>
static hipError_t skinny_split(const GemmArgs &a, const half_t *W, const half_t *X, hipStream_t s, bool reduce = true)
{
    const int kind = a.ep.kind;
    if ((kind != EP_RESID && kind != EP_STORE && kind != EP_QKV) || !a.ep.part || (a.K >> 5) % SPL ||
        (a.N / 16) % TPB || a.N % 16 || (int64_t)SPL * a.M * a.N > kSplitMaxFloats)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemm_skinny_kernel<8, U, TPB, TWO, false, false, true, PF, true, SPL>), dim3(a.N / 16 / TPB, SPL),
                       dim3(512), 0, s, W, X, 0, a.M, a.N, a.K, a.ep, (const half_t *)nullptr, 0.f,
                       (const int32_t *)nullptr, 0, (half_t *)nullptr);
    if (SPL == 1 || !reduce) return hipGetLastError();  // epilogue applied by the product / left to the caller
    const int64_t n4 = (int64_t)a.M * a.N / 4;
    const dim3 grid((unsigned)((n4 + 255) / 256));
    if (kind == EP_RESID) hipLaunchKernelGGL(split_reduce_kernel<EP_RESID>, grid, dim3(256), 0, s, SPL, a.M, a.N, a.ep);
    else if (kind == EP_QKV) hipLaunchKernelGGL(split_reduce_kernel<EP_QKV>, grid, dim3(256), 0, s, SPL, a.M, a.N, a.ep);
    else hipLaunchKernelGGL(split_reduce_kernel<EP_STORE>, grid, dim3(256), 0, s, SPL, a.M, a.N, a.ep);
    return hipGetLastError();
}

// One skinny launch: N/16/TPB work-groups of eight waves; the weight stream is
// read non-temporally (measured on every decode shape: 5-17% faster than
// cached loads, with the same HBM bytes).
template <int U, int TPB, bool TWO, bool STAGE, bool NORM, bool XT, bool PF, int NW = 8>
static void skinny(const GemmArgs &a, const half_t *W, const half_t *X, int64_t ldx, size_t lds, hipStream_t s)
{
    hipLaunchKernelGGL((gemm_skinny_kernel<NW, U, TPB, TWO, STAGE, NORM, XT, PF, true>), dim3(a.N / 16 / TPB), dim3(NW * 64),
                       lds, s, W, X, ldx, a.M, a.N, a.K, a.ep, (const half_t *)a.norm_w, a.eps, a.gather_tok,
                       a.gather_ld, (half_t *)a.gather_out);
}

hipError_t launch_gemm_f16(const GemmArgs &a, hipStream_t s)
{
    if (a.pending) *a.pending = 0;
    if (a.M <= 0) return hipSuccess;
    const half_t *W = (const half_t *)a.W, *X = (const half_t *)a.X, *nw = (const half_t *)a.norm_w;
    if (nw && !skinny_can_normalise(a.M, a.K)) return hipErrorInvalidValue;
    if (a.gather_tok && (!nw || a.x_lay != ACT_ROWS)) return hipErrorInvalidValue;  // the staged, normalising form only
    const int tiles = a.N / 16;
    // Work-group shapes below were chosen per product from cold-weight graph
    // replays of every decode shape (one row: 7B; 8 rows: 13B; 32 rows: 7B and
    // 70B).  PF (two weight rounds in flight per wave) pays where there are
    // few work-groups.
    if (a.x_lay == 1) {
        // fragment-major activations, 3..16 rows
        if (nw || a.M > 16) return hipErrorInvalidValue;
        if (a.pending && a.ep.part && a.ep.kind == EP_RESID && tiles == 320 && (a.K >> 5) % 4 == 0 &&
            (int64_t)4 * a.M * a.N <= kSplitMaxFloats) {
            // 320 row blocks (13B wo, w2), only when the next normalisation
            // adds the partials: 64 groups of five row blocks over a quarter
            // of K each, one work-group per CU, a quarter of the activation
            // block through each (8 rows: w2 26.8 -> 23.0 us, wo 11.4 ->
            // 10.0 us; two row blocks per work-group unsplit leave 96 CUs idle)
            *a.pending = 4;
            return skinny_split<4, 5, false, 4, false>(a, W, X, s, false);
        }
        if (tiles < 1024 && tiles % 2 == 0)
            skinny<8, 2, false, false, false, true, false>(a, W, X, 0, 0, s);
        else if (tiles % 4 == 0)
            skinny<2, 4, false, false, false, true, false>(a, W, X, 0, 0, s);
        else
            skinny<8, 1, false, false, false, true, false>(a, W, X, 0, 0, s);
        return hipGetLastError();
    }
    if (a.x_lay == 2) {
        // fragment-major activations, 17..32 rows (two 16-row halves)
        if (nw || a.M > 32) return hipErrorInvalidValue;
        if (a.ep.part && a.ep.kind == EP_RESID && a.K >= 16384 && tiles >= 512 && tiles % 8 == 0 &&
            (a.K >> 5) % 4 == 0 && (int64_t)4 * a.M * a.N <= kSplitMaxFloats) {
            // long residual products (70B w2): eight row blocks per work-group
            // over a quarter of K, a quarter of the activation block through
            // each CU, then a reduce launch in split order (85 -> 75 us; 72 us
            // when the next normalisation adds the partials)
            if (a.pending) *a.pending = 4;
            return skinny_split<1, 8, false, 4>(a, W, X, s, !a.pending);
        }
        if (a.pending && a.ep.part && a.ep.kind == EP_RESID && tiles == 256 && (int64_t)4 * a.M * a.N <= kSplitMaxFloats) {
            // 256 row blocks (7B wo, w2) only when the next normalisation adds
            // the partials (a reduce launch of their own costs more than the
            // split gains): four row blocks over a quarter of K for long K
            // (w2: 22.8 -> 18.3 us), else two over half of K (wo: 10.3 -> 9.0 us)
            if (a.K >= 8192 && (a.K >> 5) % 4 == 0) {
                *a.pending = 4;
                return skinny_split<2, 4, false, 4>(a, W, X, s, false);
            }
            if ((a.K >> 5) % 2 == 0) {
                *a.pending = 2;
                return skinny_split<2, 2, true, 2>(a, W, X, s, false);
            }
        }
        if (a.ep.part && a.ep.kind == EP_QKV && tiles % 5 == 0 && tiles / 5 == 128 && (a.K >> 5) % 2 == 0 &&
            (int64_t)2 * a.M * a.N <= kSplitMaxFloats)
            // 640 row blocks (70B wq|wk|wv): 128 groups of five over half of
            // K each, 256 work-groups instead of 160 (38.1 -> 32.6 us)
            return skinny_split<2, 5, false, 2>(a, W, X, s);
        if (tiles <= 256)
            skinny<8, 1, true, false, false, true, true>(a, W, X, 0, 0, s);
        else if (tiles <= 512 && tiles % 2 == 0)
            skinny<2, 2, true, false, false, true, true>(a, W, X, 0, 0, s);
        else if (tiles <= 768 && tiles % 3 == 0)
            // 768 row blocks (7B wq|wk|wv): three per work-group, one wave of
            // 256 work-groups instead of 192 (21.1 -> 18.9 us, same sums)
            skinny<2, 3, true, false, false, true, true>(a, W, X, 0, 0, s);
        else if (tiles < 1024 && tiles % 4 == 0)
            skinny<2, 4, true, false, false, true, true>(a, W, X, 0, 0, s);
        else if (tiles < 1536 && tiles % 2 == 0)
            // two rounds in flight (7B w1|w3: 34.5 -> 34.2 us, same sums)
            skinny<2, 2, true, false, false, true, true>(a, W, X, 0, 0, s);
        else if (tiles >= 2048 && tiles % 8 == 0)
            // eight row blocks per work-group read each activation fragment
            // once for all of them (the CUs' streaming rate, not HBM, bounds
            // these: 70B w1|w3 155 -> 145 us)
            skinny<1, 8, true, false, false, true, false>(a, W, X, 0, 0, s);
        else if (tiles % 4 == 0)
            skinny<2, 4, true, false, false, true, false>(a, W, X, 0, 0, s);
        else
            skinny<8, 1, true, false, false, true, false>(a, W, X, 0, 0, s);
        return hipGetLastError();
    }
    if (a.x_lay == ACT_TILED) {
        if (nw || a.M < 1024) return hipErrorInvalidValue;
        return launch_tile256<true>(a, s);
    }
    if (a.x_lay != ACT_ROWS) return hipErrorInvalidValue;
    if (a.M <= 2 && (int64_t)a.M * a.K * 2 <= STAGE_MAX_BYTES) {
        // one or two rows, staged (and normalised) in LDS
        const size_t lds = (size_t)a.M * a.K * 2;
        // four tiles per wave and round; sixteen waves for the products of
        // at most 256 row blocks without a normalisation (7B wo and w2: one
        // work-group per CU, 7.84 -> 7.42 and 16.38 -> 16.29 us)
        const bool pair = tiles >= 512 && tiles % 2 == 0, pf = tiles < 1024;
        if (nw) {
            if (pair && pf) skinny<4, 2, false, true, true, false, true>(a, W, X, a.ldx, lds, s);
            else if (pair) skinny<4, 2, false, true, true, false, false>(a, W, X, a.ldx, lds, s);
            else skinny<4, 1, false, true, true, false, true>(a, W, X, a.ldx, lds, s);
        } else {
            if (pair && pf) skinny<4, 2, false, true, false, false, true>(a, W, X, a.ldx, lds, s);
            else if (pair) skinny<4, 2, false, true, false, false, false>(a, W, X, a.ldx, lds, s);
            else skinny<4, 1, false, true, false, false, true, 16>(a, W, X, a.ldx, lds, s);
        }
    } else if (a.M <= 16) {
        skinny<8, 1, false, false, false, false, false>(a, W, X, a.ldx, 0, s);
    } else if (a.M <= 32) {
        // two row blocks per work-group reuse each activation fragment twice
        if (tiles % 2 == 0)
            skinny<4, 2, true, false, false, false, false>(a, W, X, a.ldx, 0, s);
        else
            skinny<4, 1, true, false, false, false, false>(a, W, X, a.ldx, 0, s);
    } else if (a.M < 1024) {
        int NB = (a.N + BIG_BN - 1) / BIG_BN, MB = (a.M + BIG_BM - 1) / BIG_BM;
        hipLaunchKernelGGL(gemm_big_kernel, dim3(NB * MB), dim3(256), 0, s, W, X, a.ldx, a.M, a.N, a.K, a.ep);
    } else {
        return launch_tile256<false>(a, s);
    }
    return hipGetLastError();
}

hipError_t launch_linear_f32(const GemmArgs &a, hipStream_t s)
{
    if (a.M <= 0) return hipSuccess;
    int units = (a.ep.kind == EP_QKV || a.ep.kind == EP_SWIGLU) ? a.N / 2 : a.N;
    hipLaunchKernelGGL(linear_f32_kernel, dim3((units + 63) / 64, a.M), dim3(64), 0, s,
                       (const float *)a.W, (const float *)a.X, a.ldx, a.M, a.N, a.K, a.ep);
    return hipGetLastError();
}
