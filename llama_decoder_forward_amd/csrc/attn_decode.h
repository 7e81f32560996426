// Decode attention of one (batch row, KV head) pair by one work-group of NW
// waves (walkthrough section 3.5 step 5, GQA of section 3.4), the body of the
// decode attention kernel.
//
// The attended length L = pos + 1 is walked in 32-key steps, wave w taking
// steps w, w+NW, ...; each wave keeps the running max / sum / unnormalised
// output of all n_rep query heads of the group, so every K/V byte is read
// once per query group.  S^T = K Q^T and O^T = V^T P^T on
// v_mfma_f32_16x16x32_f16: the query is the MFMA column (lane % 16) and each
// lane owns its query's softmax state.  Inside a 32-key step, row r of S^T
// sub-tile t is key 8*(r/4) + 4*t + r%4, so the accumulator lane group g
// holds keys 8g..8g+7 of the step -- exactly the B-operand k-group of P^T --
// and the matching V^T operand is one contiguous 16-byte load.  A wave's first
// step (of the static cache, or inside the row's first block of a paged one) is
// loaded before the attended length arrives.  PF: a
// wave's next step is loaded while the current one computes.  PAGED: each 32-key step
// lies in one block of the row's table; the table entries the row uses are
// held in lanes and read with readlane.  NT: K and V are read non-temporally.  The NW
// waves' states are merged in one round through LDS (fixed wave order).
#pragma once
#include "common.h"

namespace adec {

__device__ __forceinline__ floatx4 mfma16(half8 a, half8 b, floatx4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Key (0..31 within a step) held in row r of sub-tile t.
__device__ __forceinline__ int perm_key(int t, int r) { return 8 * (r >> 2) + 4 * t + (r & 3); }

// NT: K and V are read with non-temporal loads
template <bool NT>
__device__ __forceinline__ half8 ld_kv(const half_t *p)
{
    if (NT) return __builtin_nontemporal_load(reinterpret_cast<const half8 *>(p));
    return *reinterpret_cast<const half8 *>(p);
}

constexpr float kNegBig = -1.0e30f;  // running-max start: finite, so exp(m_old - m_new) is never NaN

template <int NW, bool PF, bool PAGED, bool NT = false>
__device__ __forceinline__ void attn_decode_wg(const half_t *__restrict__ q, const half_t *__restrict__ kc,
                                               const half_t *__restrict__ vc, int H, int Hkv, int S, const KvPages &pg,
                                               int b, int kvh, int L, half_t *__restrict__ out, int out_lay,
                                               floatx4 (*so)[8][64], float (*sm)[16], float (*sl)[16])
// so, sm, sl: LDS for the states of all NW waves
{
    constexpr int hd = 128;
    // the wave index is uniform across the wave: in a scalar register, so the
    // step loop and its block lookups branch on scalars
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int n_rep = H / Hkv;
    const int r = lane & 15, g = lane >> 4;
    const bool qv = r < n_rep;
    const int h = kvh * n_rep + r;
    // scores in log2 units (scaled by log2(e) / sqrt(d)): each softmax term
    // is one native exp2, as in the prefill kernel
    const float sl2 = 1.4426950408889634f / sqrtf((float)hd);
    const int nsteps = (L + 31) / 32;
    const half8 z = {};

    half8 qb[4];
    const half_t *qrow = q + ((int64_t)b * H + (qv ? h : 0)) * hd;
#pragma unroll
    for (int s = 0; s < 4; s++)
        qb[s] = qv ? *reinterpret_cast<const half8 *>(qrow + 32 * s + 8 * g) : z;

    // PAGED: lane j holds entries j and 64 + j of the row's block table (the
    // entries its L positions use), so a step finds its block with a lane
    // read instead of a memory load; entries from 128 on are loaded
    // (loaded after the early first step below, which does not need them)
    int tv0 = 0, tv1 = 0;
    auto load_table = [&]() {
        const int *trow = pg.tab + (int64_t)b * pg.ld;
        const int nent = ((L - 1) >> pg.shift) + 1;
        tv0 = lane < nent ? trow[lane] : 0;
        tv1 = 64 + lane < nent ? trow[64 + lane] : 0;
    };
    // element offset of the first key of 32-key step st in both K and V
    auto step_base = [&](int st) -> int64_t {
        const int k0 = 32 * st;
        if (PAGED) {
            const int e = k0 >> pg.shift;
            int64_t blk;
            if (e < 64) blk = __builtin_amdgcn_readlane(tv0, e);
            else if (e < 128) blk = __builtin_amdgcn_readlane(tv1, e - 64);
            else blk = pg.tab[(int64_t)b * pg.ld + e];
            return (((blk * Hkv + kvh) << pg.shift) + (k0 & ((1 << pg.shift) - 1))) * hd;
        }
        return (((int64_t)b * Hkv + kvh) * S + k0) * hd;
    };

    floatx4 acc[8];
#pragma unroll
    for (int dt = 0; dt < 8; dt++) acc[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
    float mrun = kNegBig, lrun = 0.f;

    // all K and V operands of a step are loaded before any of its arithmetic
    auto load = [&](int st, int64_t base, half8 (&kf)[2][4], half8 (&vf)[8]) {
        const int k0 = 32 * st;
#pragma unroll
        for (int t = 0; t < 2; t++) {
            // the cache holds operand (t, s) of the step as 1 KiB in lane
            // order (k16_offset); keys past L read entries of the same
            // stream and are zeroed
            const bool ok = k0 + perm_key(t, r) < L;
#pragma unroll
            for (int s = 0; s < 4; s++)
                kf[t][s] = ok ? ld_kv<NT>(kc + base + ((t * 4 + s) * 64 + lane) * 8) : z;
        }
        // V: one 16-byte load per operand; entries of keys past L (the
        // step's block is always allocated in full) are zeroed, since a
        // probability of 0 times a stale non-finite value would not vanish
        const int kk = k0 + 8 * g;
        const bool vok = kk + 8 <= L;
        const half_t *vblk = vc + base + 8 * g;
#pragma unroll
        for (int dt = 0; dt < 8; dt++) {
            half8 v = ld_kv<NT>(vblk + (16 * dt + r) * 32);
            if (!vok) {
#pragma unroll
                for (int e = 0; e < 8; e++) v[e] = kk + e < L ? v[e] : (half_t)0.f;
            }
            vf[dt] = v;
        }
    };
    auto compute = [&](int st, const half8 (&kf)[2][4], const half8 (&vf)[8]) {
        const int k0 = 32 * st;
        floatx4 sc[2];
#pragma unroll
        for (int t = 0; t < 2; t++) {
            floatx4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; s++) a = mfma16(kf[t][s], qb[s], a);
            sc[t] = a;
        }
        float p[8];
        float mx = kNegBig;
#pragma unroll
        for (int t = 0; t < 2; t++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int key = k0 + 8 * g + 4 * t + i;
                float v = key < L ? sc[t][i] * sl2 : -INFINITY;
                p[4 * t + i] = v;
                mx = fmaxf(mx, v);
            }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mnew = fmaxf(mrun, mx);
        const float fac = __builtin_amdgcn_exp2f(mrun - mnew);
        float ls = 0.f;
        half8 pb;
#pragma unroll
        for (int e = 0; e < 8; e++) {
            float ev = __builtin_amdgcn_exp2f(p[e] - mnew);
            ls += ev;
            pb[e] = (half_t)ev;
        }
        ls += __shfl_xor(ls, 16);
        ls += __shfl_xor(ls, 32);
        lrun = lrun * fac + ls;
        mrun = mnew;
#pragma unroll
        for (int dt = 0; dt < 8; dt++) acc[dt] = mfma16(vf[dt], pb, acc[dt] * fac);
    };
    // static cache: a wave's first 32-key step does not depend on the
    // attended length (read from memory by the kernel), so it is loaded
    // before the length is known, and its keys past the length are zeroed
    // afterwards as load() zeroes them (same operands)
    auto load_raw = [&](int64_t base, half8 (&kf)[2][4], half8 (&vf)[8]) {
#pragma unroll
        for (int t = 0; t < 2; t++)
#pragma unroll
            for (int s = 0; s < 4; s++) kf[t][s] = ld_kv<NT>(kc + base + ((t * 4 + s) * 64 + lane) * 8);
        const half_t *vblk = vc + base + 8 * g;
#pragma unroll
        for (int dt = 0; dt < 8; dt++) vf[dt] = ld_kv<NT>(vblk + (16 * dt + r) * 32);
    };
    auto mask = [&](int st, half8 (&kf)[2][4], half8 (&vf)[8]) {
        const int k0 = 32 * st;
#pragma unroll
        for (int t = 0; t < 2; t++)
            if (!(k0 + perm_key(t, r) < L)) {
#pragma unroll
                for (int s = 0; s < 4; s++) kf[t][s] = z;
            }
        const int kk = k0 + 8 * g;
        if (!(kk + 8 <= L)) {
#pragma unroll
            for (int dt = 0; dt < 8; dt++)
#pragma unroll
                for (int e = 0; e < 8; e++) vf[dt][e] = kk + e < L ? vf[dt][e] : (half_t)0.f;
        }
    };
    half8 kf[2][4], vf[8];
    int st = wave;
    // paged: a first step inside the row's first block (table entry 0, which
    // every row holds, position 0 being written first) is read early the same way
    const bool spec = PAGED ? 32 * (wave + 1) <= (1 << pg.shift) : (wave + 1) * 32 <= S;
    if (spec) {
        int64_t sb;
        if (PAGED) {
            const int64_t blk = pg.tab[(int64_t)b * pg.ld];
            sb = (((blk * Hkv + kvh) << pg.shift) + 32 * st) * hd;
        } else {
            sb = step_base(st);
        }
        load_raw(sb, kf, vf);
    }
    if (PAGED) load_table();
    if (spec) {
        if (st < nsteps) mask(st, kf, vf);
    } else if (st < nsteps) {
        load(st, step_base(st), kf, vf);
    }
    for (; st < nsteps; st += NW) {
        const int nx = st + NW;
        const int64_t nbase = nx < nsteps ? step_base(nx) : 0;
        if (PF) {
            half8 kn[2][4], vn[8];
            if (nx < nsteps) load(nx, nbase, kn, vn);
            compute(st, kf, vf);
#pragma unroll
            for (int t = 0; t < 2; t++)
#pragma unroll
                for (int s = 0; s < 4; s++) kf[t][s] = kn[t][s];
#pragma unroll
            for (int dt = 0; dt < 8; dt++) vf[dt] = vn[dt];
        } else {
            compute(st, kf, vf);
            if (nx < nsteps) load(nx, nbase, kf, vf);
        }
    }

    // merge in one round: every wave hands its state to LDS; after one
    // barrier wave w combines the column blocks dt = w, w + NW, ... over all
    // waves in wave order and stores them (lane (r, g) holds
    // O^T[16 dt + 4 g + i][head r])
#pragma unroll
    for (int dt = 0; dt < 8; dt++) so[wave][dt][lane] = acc[dt];
    if (g == 0) {
        sm[wave][r] = mrun;
        sl[wave][r] = lrun;
    }
    __syncthreads();
    float M = sm[0][r];
#pragma unroll
    for (int w = 1; w < NW; w++) M = fmaxf(M, sm[w][r]);
    float fw[NW], l = 0.f;
#pragma unroll
    for (int w = 0; w < NW; w++) {
        fw[w] = __builtin_amdgcn_exp2f(sm[w][r] - M);
        l += sl[w][r] * fw[w];
    }
    const float inv = 1.0f / l;
    for (int dt = wave; dt < 8; dt += NW) {
        floatx4 o = so[0][dt][lane] * fw[0];
#pragma unroll
        for (int w = 1; w < NW; w++) o += so[w][dt][lane] * fw[w];
        if (qv) {
            half4 hv;
            for (int i = 0; i < 4; i++) hv[i] = (half_t)(o[i] * inv);
            const int c = 16 * dt + 4 * g;  // 4 consecutive columns inside one 8-column group
            half_t *orow = out + ((int64_t)b * H + h) * hd;
            if (out_lay) *reinterpret_cast<half4 *>(out + act_offset(b, (int64_t)h * hd + c, (int64_t)H * hd, 0, out_lay)) = hv;
            else *reinterpret_cast<half4 *>(orow + c) = hv;
        }
    }
}

}  // namespace adec
