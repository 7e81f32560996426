// Scaled dot-product attention over the static KV cache (walkthrough
// section 3.5 step 5): scores q.k / sqrt(d), the causal mask of section 3.8
// (query at position p sees keys 0..p), softmax in fp32 with the maximum
// subtracted, weighted sum of values; query head h reads KV head h / n_rep
// (repeat_kv, section 3.4).
//
// Cache layout (per layer): streams of positions per (block, KV head), K
// key-major, V in blocks of 32 keys, d-major inside a block (common.h); a
// static cache has one stream per (row, KV head), a paged one reaches a
// row's positions through its block table.  Both kernels compute S^T = K Q^T and O^T = V^T P^T with
// v_mfma_f32_16x16x32_f16, so the query is the MFMA column (lane % 16) and
// each lane owns its query's running max / sum with no cross-lane moves.
//
// Key permutation: inside a 32-key step, row r of S^T sub-tile t (t = 0, 1)
// is key 8*(r/4) + 4*t + r%4.  The accumulator lane group g then holds keys
// 8g..8g+7 of the step, which is exactly the B-operand k-group of P^T, and
// the matching A operand V^T[d][8g..8g+7] is one contiguous 16-byte load.
#include <type_traits>

#include "common.h"
#include "attn_decode.h"

namespace {

__device__ __forceinline__ floatx4 mfma16(half8 a, half8 b, floatx4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}


constexpr float kNegBig = -1.0e30f;  // running-max start: finite, so exp(m_old - m_new) is never NaN

// Maximum and sum over the four 16-lane rows of a wave, every lane keeping its
// column (the query), by gfx950's row swaps (no LDS round trip).  Every row
// ends with the same bits; the sum is (x0 + x1) + (x2 + x3).
__device__ __forceinline__ float vmax(float a, float b)
{
    float d;
    asm("v_max_f32 %0, %1, %2" : "=v"(d) : "v"(a), "v"(b));
    return d;
}
// a product the compiler may not fuse with a following add (scores are
// scaled and rounded before the maximum is subtracted, in every tile alike)
__device__ __forceinline__ float mul_rn(float a, float b)
{
#pragma clang fp contract(off)
    return a * b;
}
__device__ __forceinline__ float rows_max(float v)
{
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = vmax(__uint_as_float(a[0]), __uint_as_float(a[1]));
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return vmax(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows_sum(float v)
{
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// ---------------------------------------------------------------------------
// Decode: one work-group of NW waves per (row b, KV head).  The attended
// length L = pos + 1 is walked in 32-key steps, wave w taking steps w, w+NW,
// ...; each wave keeps the running max / sum / unnormalised output of all
// n_rep query heads of the group, so every K/V byte is read once per query
// group.  PF: a wave's next step is loaded while the current one computes.
// The NW waves are merged in LDS in one round (fixed order), and the
// normalised output written.  Few (row, KV head) pairs take 8 waves (the
// work-group count, not the bandwidth, is the limit there); many pairs
// take 2 or 4 so that more of them fit the CUs at once.  PAGED: each 32-key
// step lies in one block of the row's table (blocks hold a multiple of 32
// positions); the block id of a wave's next step is read before the current
// step computes.
// ---------------------------------------------------------------------------
template <int NW, bool PF, bool PAGED, bool NT = false>
__global__ __launch_bounds__(NW * 64) void attn_decode_kernel(
    const half_t *__restrict__ q, const half_t *__restrict__ kc, const half_t *__restrict__ vc,
    int H, int Hkv, int S, KvPages pg, const int *pos_dev, int pos_imm, const int *pos_rows,
    half_t *__restrict__ out, int out_lay)
{
    __shared__ floatx4 so[NW][8][64];
    __shared__ float sm[NW][16], sl[NW][16];
    const int bk = blockIdx.x, b = bk / Hkv, kvh = bk % Hkv;
    const int L = (pos_rows ? pos_rows[b] : (pos_dev ? *pos_dev : pos_imm)) + 1;
    adec::attn_decode_wg<NW, PF, PAGED, NT>(q, kc, vc, H, Hkv, S, pg, b, kvh, L, out, out_lay, so, sm, sl);
}

// ---------------------------------------------------------------------------
// Causal prefill of T tokens at positions p0..p0+T-1 of every row over the
// cache prefix 0..p0-1 and themselves (walkthrough section 3.8: a zero
// block before the causal triangle when p0 > 0): flash-style online
// softmax.  One work-group per (row, head, 128 queries): 4 waves x 32
// queries (two MFMA column groups), two work-groups per CU.  64-key tiles of
// K (in permuted operand order) and V^T reach LDS by direct global -> LDS
// copies into a two-stage ring, the next tile in flight while the current
// one computes.  Tiles entirely above a wave's last query are skipped; tiles
// that reach past its first query are masked.  Each 32-key half of a tile
// lies in one cache stream (blocks of a paged cache hold a multiple of 32
// positions), located once per tile.
// ---------------------------------------------------------------------------
constexpr int PF_Q = 128, PF_K = 64;

constexpr int PF_LDS = 2 * 2 * PF_K * 128 * 2;  // two stages of a K and a V tile (bytes)
constexpr bool HEAVY_FIRST = true;

__global__ __launch_bounds__(256, 2) void attn_prefill_kernel(const half_t *__restrict__ q,
                                                           const half_t *__restrict__ kc,
                                                           const half_t *__restrict__ vc, int Tu, int p0u,
                                                           int H, int Hkv, int S, KvPages pg, const int *cu,
                                                           half_t *__restrict__ out, int out_lay, int ny)
{
    const int hd = 128;
    extern __shared__ half8 smem[];
    // per stage: K tile as 4 sub-tiles x 4 d-steps x 64 lanes, V^T tile as 8
    // d-tiles x 2 key-steps x 64 lanes (operand order)
    half8 *const klds = smem, *const vlds = smem + 2 * PF_K * hd / 8;
    // Work order.  Work-groups are dealt to the eight XCDs in turn (group i
    // to XCD i % 8), each XCD with its own L2.  GQA (n_rep > 1), when the
    // grid divides evenly: every XCD takes a contiguous range of a work list
    // that runs (row, KV head) group by group, query tiles from the last
    // (the longest) down, the n_rep query heads innermost, so the work-groups
    // that read one K/V stream run together on one XCD.  Otherwise query
    // tile by query tile (HEAVY_FIRST: the longest first), every (row, head)
    // inside one: with B * H a multiple of 8 each (row, head) then stays on
    // one XCD (measured: 13B, one head per KV head, lost 20% to the
    // contiguous ranges).
    const int nbh = (int)gridDim.x / ny, n_rep = H / Hkv;
    int b, h, qt;
    if (n_rep > 1 && (gridDim.x & 7) == 0) {
        const int w = ((int)blockIdx.x & 7) * (int)(gridDim.x >> 3) + ((int)blockIdx.x >> 3);
        const int hh = w % n_rep, yk = (w / n_rep) % ny, grp = w / (n_rep * ny);
        b = grp / Hkv;
        h = (grp % Hkv) * n_rep + hh;
        qt = ny - 1 - yk;
    } else {
        const int yk = (int)blockIdx.x / nbh, rem = (int)blockIdx.x % nbh;
        b = rem / H;
        h = rem % H;
        qt = HEAVY_FIRST ? ny - 1 - yk : yk;
    }
    // uniform rows: T = Tu tokens at p0u..; varlen: row b's T tokens are the
    // packed rows cu[b].. at positions 0..
    int T = Tu, p0 = p0u;
    int64_t rbase = (int64_t)b * Tu;
    if (cu) {
        rbase = cu[b];
        T = cu[b + 1] - cu[b];
        p0 = 0;
    }
    if (qt * PF_Q >= T) return;  // a query tile past this row's end (whole work-group)
    const int kvh = h / (H / Hkv);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r = lane & 15, g = lane >> 4;
    const int q0 = qt * PF_Q;
    const int wq0 = q0 + 32 * wave;  // this wave's first query
    // scores are kept in log2 units (scaled by log2(e) / sqrt(d)), so each
    // softmax term is one native exp2: exp(s / sqrt(d) - m) = 2^(s log2(e) /
    // sqrt(d) - m log2(e))
    const float sl2 = 1.4426950408889634f / sqrtf((float)hd);
    const half8 z = {};

    half8 qb[2][4];
#pragma unroll
    for (int c = 0; c < 2; c++) {
        const int t = wq0 + 16 * c + r;
        const half_t *qrow = q + ((rbase + (t < T ? t : 0)) * H + h) * hd;
#pragma unroll
        for (int s = 0; s < 4; s++)
            qb[c][s] = t < T ? *reinterpret_cast<const half8 *>(qrow + 32 * s + 8 * g) : z;
    }

    // element offset of key k0 (a multiple of 32) in both K and V
    auto key_base = [&](int k0) -> int64_t {
        int off;
        const int64_t st = kv_stream(pg, b, kvh, k0, Hkv, off);
        return k_offset(st, off, 0, S, hd);
    };

    floatx4 acc[2][8];
#pragma unroll
    for (int c = 0; c < 2; c++)
#pragma unroll
        for (int dt = 0; dt < 8; dt++) acc[c][dt] = floatx4{0.f, 0.f, 0.f, 0.f};
    float mrun[2] = {kNegBig, kNegBig}, lrun[2] = {0.f, 0.f};

    // query t sits at absolute position p0 + t and sees keys 0 .. p0 + t
    // (the cache prefix written before, then the causal block)
    const int Lk = p0 + T;
    const int qlast = min(q0 + PF_Q, T) - 1;
    const int ntiles = (p0 + qlast) / PF_K + 1;

    // Stage kt of the tile ring: direct global -> LDS copies, each lane
    // fetching the 16 bytes that belong at its slot of the operand order.
    // Wave w copies K blocks 4w..4w+3 (block (ks, t, s): lane rr + 16 gg
    // holds key 32 ks + 8 (rr / 4) + 4 t + rr % 4, d 32 s + 8 gg .. +7; the
    // cache stores each such block as 1 KiB in this order, k16_offset) and V
    // blocks 4w..4w+3 (block (dt, ks): lane d % 16 + 16 gg holds the keys
    // 32 ks + 8 gg .. +7 of dimension d = 16 dt + d % 16).  Keys past Lk read
    // cache entries of the same (row, KV head) that the scores mask out.
    auto issue_tile = [&](int kt) {
        const int base = kt * PF_K, buf = kt & 1;
        // base < Lk for every tile walked; the second half only when in range
        const int64_t hb0 = key_base(base);
        const int64_t hb1 = base + 32 < Lk ? key_base(base + 32) : hb0;
        const int rr = lane & 15, gg = lane >> 4;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int blk = 4 * wave + j;
            const int ks = blk >> 3, ts = blk & 7;  // (t, s) block of the 32-key half ks
            lds_copy16(kc + (ks ? hb1 : hb0) + (ts * 64 + lane) * 8, klds + (buf * 16 + blk) * 64);
        }
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int blk = 4 * wave + j;
            const int dt = blk >> 1, ks = blk & 1;
            lds_copy16(vc + (ks ? hb1 : hb0) + (16 * dt + rr) * 32 + gg * 8, vlds + (buf * 16 + blk) * 64);
        }
    };
    // V entries past Lk get probability 0, but 0 times a non-finite stale
    // value would not vanish: after its copies of the tile holding Lk have
    // landed, each lane zeroes the keys past Lk in its own V slots
    auto clear_v_tail = [&](int kt) {
        const int base = kt * PF_K, buf = kt & 1, gg = lane >> 4;
        if (base + PF_K <= Lk) return;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int blk = 4 * wave + j, ks = blk & 1;
            const int key0 = base + 32 * ks + 8 * gg;
            if (key0 + 8 > Lk) {
                half8 &slot = vlds[(buf * 16 + blk) * 64 + lane];
                half8 v = slot;
#pragma unroll
                for (int e = 0; e < 8; e++) v[e] = key0 + e < Lk ? v[e] : (half_t)0.f;
                slot = v;
            }
        }
    };

    // One 64-key tile: S^T for both query column groups (every K fragment is
    // read from LDS once and used for both), the online softmax, and
    // O^T += V^T P^T (every V fragment read once).  MASKED: the causal mask
    // (only tiles that reach past this wave's first query need it).
    auto step = [&](const half8 *kl, const half8 *vl, int kbase, auto masked_c) {
        constexpr bool MASKED = decltype(masked_c)::value;
        floatx4 sc[2][2][2];  // [c][ks][t]
#pragma unroll
        for (int ks = 0; ks < 2; ks++)
#pragma unroll
            for (int t = 0; t < 2; t++) {
                half8 kf[4];
#pragma unroll
                for (int s = 0; s < 4; s++) kf[s] = kl[((ks * 2 + t) * 4 + s) * 64 + lane];
#pragma unroll
                for (int c = 0; c < 2; c++) {
                    floatx4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s < 4; s++) a = mfma16(kf[s], qb[c][s], a);
                    sc[c][ks][t] = a;
                }
            }
        half8 pb[2][2];
        float fac[2];
#pragma unroll
        for (int c = 0; c < 2; c++) {
            const int qi = p0 + wq0 + 16 * c + r;  // this lane's query position
            float p[2][8];
            float mx = kNegBig;
#pragma unroll
            for (int ks = 0; ks < 2; ks++)
#pragma unroll
                for (int t = 0; t < 2; t++)
#pragma unroll
                    for (int i = 0; i < 4; i++) {
                        float v = mul_rn(sc[c][ks][t][i], sl2);
                        if (MASKED && kbase + 32 * ks + 8 * g + 4 * t + i > qi) v = -INFINITY;
                        p[ks][4 * t + i] = v;
                        mx = fmaxf(mx, v);
                    }
            const float mnew = fmaxf(mrun[c], rows_max(mx));
            fac[c] = __builtin_amdgcn_exp2f(mrun[c] - mnew);
            float ls = 0.f;
#pragma unroll
            for (int ks = 0; ks < 2; ks++)
#pragma unroll
                for (int e = 0; e < 8; e++) {
                    const float ev = __builtin_amdgcn_exp2f(p[ks][e] - mnew);
                    ls += ev;
                    pb[c][ks][e] = (half_t)ev;
                }
            lrun[c] = lrun[c] * fac[c] + rows_sum(ls);
            mrun[c] = mnew;
        }
        // the rescale by a factor of exactly 1 (no lane's maximum moved) is
        // skipped: the same bits
        if (__any(fac[0] != 1.f || fac[1] != 1.f)) {
#pragma unroll
            for (int dt = 0; dt < 8; dt++) {
                acc[0][dt] = acc[0][dt] * fac[0];
                acc[1][dt] = acc[1][dt] * fac[1];
            }
        }
#pragma unroll
        for (int dt = 0; dt < 8; dt++) {
#pragma unroll
            for (int ks = 0; ks < 2; ks++) {
                const half8 vf = vl[(dt * 2 + ks) * 64 + lane];
                acc[0][dt] = mfma16(vf, pb[0][ks], acc[0][dt]);
                acc[1][dt] = mfma16(vf, pb[1][ks], acc[1][dt]);
            }
        }
    };

    issue_tile(0);
    for (int kt = 0; kt < ntiles; kt++) {
        // this wave's copies of stage kt have landed (none of stage kt+1 is
        // issued yet); the barrier makes every wave's visible and ends the
        // reads of stage kt-1, whose buffer the next copies reuse
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        clear_v_tail(kt);
        __syncthreads();
        if (kt + 1 < ntiles) issue_tile(kt + 1);
        const half8 *kl = klds + (kt & 1) * 1024, *vl = vlds + (kt & 1) * 1024;
        const int kbase = kt * PF_K;
        if (kbase > p0 + wq0 + 31) continue;  // all keys after this wave's queries
        // tiles wholly before this wave's first query need no causal mask
        // (a uniform test; the two forms are separate code)
        if (kbase + PF_K - 1 <= p0 + wq0) step(kl, vl, kbase, std::false_type{});
        else step(kl, vl, kbase, std::true_type{});
    }
#pragma unroll
    for (int c = 0; c < 2; c++) {
        const int t = wq0 + 16 * c + r;
        if (t >= T) continue;
        const float inv = 1.0f / lrun[c];
        half_t *orow = out + ((rbase + t) * H + h) * hd;
#pragma unroll
        for (int dt = 0; dt < 8; dt++) {
            half4 o;
#pragma unroll
            for (int i = 0; i < 4; i++) o[i] = (half_t)(acc[c][dt][i] * inv);
            const int col = 16 * dt + 4 * g;  // 4 consecutive columns inside one 8-column group
            if (out_lay)
                *reinterpret_cast<half4 *>(out + act_offset((int)(rbase + t), (int64_t)h * hd + col, (int64_t)H * hd, 0, out_lay)) = o;
            else
                *reinterpret_cast<half4 *>(orow + col) = o;
        }
    }
}

// ---------------------------------------------------------------------------
// fp32 models (small): one work-group per (b, h, query), scores in LDS.
// ---------------------------------------------------------------------------
__global__ void attn_f32_kernel(const float *q, const float *kc, const float *vc, int T, int H,
                                int Hkv, int hd, int Sb, KvPages pg, const int *pos_dev, int pos_imm,
                                const int *pos_rows, const int *cu, float *out)
{
    extern __shared__ float sh[];  // L scores
    const int bh = blockIdx.x, b = bh / H, h = bh % H, t = blockIdx.y;
    const int kvh = h / (H / Hkv);
    // query row and position: uniform rows, per-row decode positions, or
    // varlen rows packed at cu[b].. (positions 0..)
    int64_t row = (int64_t)b * T + t;
    int pos = (pos_dev ? *pos_dev : pos_imm) + t;
    if (pos_rows) pos = pos_rows[b];
    if (cu) {
        if (t >= cu[b + 1] - cu[b]) return;  // whole work-group
        row = cu[b] + t;
        pos = t;
    }
    const int L = pos + 1;
    const float *qr = q + (row * H + h) * hd;
    const float scale = 1.0f / sqrtf((float)hd);
    for (int j = threadIdx.x; j < L; j += blockDim.x) {
        int off;
        const int64_t st = kv_stream(pg, b, kvh, j, Hkv, off);
        const float *kr = kc + k_offset(st, off, 0, Sb, hd);
        float s = 0.f;
        for (int d = 0; d < hd; d++) s = fmaf(qr[d], kr[d], s);
        sh[j] = s * scale;
    }
    __syncthreads();
    float mx = -INFINITY;
    for (int j = 0; j < L; j++) mx = fmaxf(mx, sh[j]);
    float sum = 0.f;
    for (int j = 0; j < L; j++) sum += expf(sh[j] - mx);
    for (int d = threadIdx.x; d < hd; d += blockDim.x) {
        float o = 0.f;
        for (int j = 0; j < L; j++) {
            int off;
            const int64_t st = kv_stream(pg, b, kvh, j, Hkv, off);
            o = fmaf(expf(sh[j] - mx) / sum, vc[v32_offset(st, off, d, Sb, hd)], o);
        }
        out[(row * H + h) * hd + d] = o;
    }
}

template <typename Tv>
__global__ void kv_write_kernel(const Tv *k, const Tv *v, int T, int pos0, int Hkv, int hd, int Sb,
                                KvPages pg, Tv *kc, Tv *vc)
{
    // one thread per element of k[B][T][Hkv][hd]
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t per_row = (int64_t)T * Hkv * hd;
    const int b = (int)(blockIdx.y);
    if (i >= per_row) return;
    const int d = (int)(i % hd), kvh = (int)((i / hd) % Hkv), t = (int)(i / ((int64_t)hd * Hkv));
    const int pos = pos0 + t;
    int off;
    const int64_t st = kv_stream(pg, b, kvh, pos, Hkv, off);
    kc[sizeof(Tv) == 2 ? k16_offset(st, off, d, Sb, hd) : k_offset(st, off, d, Sb, hd)] = k[(int64_t)b * per_row + i];
    if (sizeof(Tv) == 2)
        vc[v16_offset(st, off, d, Sb, hd)] = v[(int64_t)b * per_row + i];
    else
        vc[v32_offset(st, off, d, Sb, hd)] = v[(int64_t)b * per_row + i];
}

}  // namespace

template <bool PAGED>
hipError_t launch_decode(const AttnArgs &a, hipStream_t s)
{
    const int pairs = a.B * a.Hkv;
    const half_t *q = (const half_t *)a.q, *kc = (const half_t *)a.kcache, *vc = (const half_t *)a.vcache;
    half_t *o = (half_t *)a.out;
    if (pairs >= 512)  // non-temporal K/V loads: 7B bs32 30.9 -> 29.6 us (L = 204), 51.9 -> 48.5 us (L = 512)
        hipLaunchKernelGGL((attn_decode_kernel<2, true, PAGED, true>), dim3(pairs), dim3(128), 0, s, q, kc, vc, a.H,
                           a.Hkv, a.Sb, a.pg, a.pos_dev, a.pos_imm, a.pos_rows, o, a.out_lay);
    else if (pairs >= 300)  // 320 pairs (13B bs8; 256 (70B bs32) do better with eight): non-temporal K/V
                            // loads, 13B bs8 decode attention 2.22 -> 2.05 ms per step
        hipLaunchKernelGGL((attn_decode_kernel<4, false, PAGED, true>), dim3(pairs), dim3(256), 0, s, q, kc, vc, a.H,
                           a.Hkv, a.Sb, a.pg, a.pos_dev, a.pos_imm, a.pos_rows, o, a.out_lay);
    else if (pairs >= 128)  // non-temporal K/V loads: 7% faster on 256 pairs (70B bs32), slower elsewhere
        hipLaunchKernelGGL((attn_decode_kernel<8, false, PAGED, true>), dim3(pairs), dim3(512), 0, s, q, kc, vc, a.H,
                           a.Hkv, a.Sb, a.pg, a.pos_dev, a.pos_imm, a.pos_rows, o, a.out_lay);
    else  // next step prefetched: 7B bs1 decode attention 0.348 -> 0.322 ms per step
        hipLaunchKernelGGL((attn_decode_kernel<8, true, PAGED>), dim3(pairs), dim3(512), 0, s, q, kc, vc, a.H, a.Hkv,
                           a.Sb, a.pg, a.pos_dev, a.pos_imm, a.pos_rows, o, a.out_lay);
    return hipGetLastError();
}

hipError_t launch_attn_decode_f16(const AttnArgs &a, hipStream_t s)
{
    if (a.out_lay && (a.out_lay > 2 || a.B > 16 * a.out_lay || a.T != 1)) return hipErrorInvalidValue;
    return a.pg.tab ? launch_decode<true>(a, s) : launch_decode<false>(a, s);
}

hipError_t launch_attn_prefill_f16(const AttnArgs &a, hipStream_t s)
{
    if (a.out_lay != ACT_ROWS && a.out_lay != ACT_TILED) return hipErrorInvalidValue;
    const int ny = (a.T + PF_Q - 1) / PF_Q;
    hipLaunchKernelGGL(attn_prefill_kernel, dim3(a.B * a.H * ny), dim3(256), PF_LDS, s, (const half_t *)a.q,
                       (const half_t *)a.kcache, (const half_t *)a.vcache, a.T, a.pos_imm, a.H, a.Hkv, a.Sb,
                       a.pg, a.cu, (half_t *)a.out, a.out_lay, ny);
    return hipGetLastError();
}

hipError_t launch_attn_f32(const AttnArgs &a, hipStream_t s)
{
    size_t sh = sizeof(float) * (size_t)a.S;
    hipLaunchKernelGGL(attn_f32_kernel, dim3(a.B * a.H, a.T), dim3(64), sh, s, (const float *)a.q,
                       (const float *)a.kcache, (const float *)a.vcache, a.T, a.H, a.Hkv, a.hd,
                       a.Sb, a.pg, a.pos_dev, a.pos_imm, a.pos_rows, a.cu, (float *)a.out);
    return hipGetLastError();
}

hipError_t launch_kv_write(const void *k, const void *v, int B, int T, int pos0, int Hkv, int hd,
                           int Sb, const KvPages &pg, int dtype, void *kcache, void *vcache, hipStream_t s)
{
    int64_t per_row = (int64_t)T * Hkv * hd;
    dim3 grid((unsigned)((per_row + 255) / 256), B);
    if (dtype == 1)
        hipLaunchKernelGGL(kv_write_kernel<half_t>, grid, dim3(256), 0, s, (const half_t *)k,
                           (const half_t *)v, T, pos0, Hkv, hd, Sb, pg, (half_t *)kcache, (half_t *)vcache);
    else
        hipLaunchKernelGGL(kv_write_kernel<float>, grid, dim3(256), 0, s, (const float *)k,
                           (const float *)v, T, pos0, Hkv, hd, Sb, pg, (float *)kcache, (float *)vcache);
    return hipGetLastError();
}
