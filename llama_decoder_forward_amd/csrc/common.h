// Internal definitions shared by the HIP kernels and the host library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef _Float16 half_t;
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Weight layout
//
// fp16 matrices W[N][K] (logical out x in) are stored as 16 x 32 tiles of
// 512 halves (1 KiB).  Tile (nt, kt) starts at (nt * K/32 + kt) * 512; inside
// it, the 8 halves of lane l (l = 0..63) are W[16 nt + l%16][32 kt + 8 (l/16)
// + e], e = 0..7, at offset 8 l.  This is the A-operand layout of
// v_mfma_f32_16x16x32_f16, so one 16-byte load per lane fetches an MFMA
// operand and a wave's 1 KiB load is contiguous.
// fp32 matrices are plain row-major.
// ---------------------------------------------------------------------------
__host__ __device__ inline int64_t tiled_offset(int64_t n, int64_t k, int64_t K)
{
    int64_t nt = n >> 4, kt = k >> 5;
    int64_t lane = (n & 15) + 16 * ((k & 31) >> 3);
    return (nt * (K >> 5) + kt) * 512 + lane * 8 + (k & 7);
}

// KV cache (per layer).  The cache is a set of "streams" of Sb positions,
// one per (block, KV head), stream index blk * Hkv + kvh:
//  - static cache: block b is batch row b and Sb = max_seq_len;
//  - paged cache (nano-vllm notes, allocate_kv_cache): a pool of blocks of
//    Sb = bs positions (a power of two >= 32); position p of row b lives in
//    block tab[b * ld + p / bs] at offset p % bs.
// Inside a stream, fp16 models use
//   K[s][d]            key-major: a key's 128 values are contiguous;
//   V[s/32][d][s%32]   blocks of 32 keys, d-major inside a block, so a
//                      32-key step reads one contiguous 8 KiB block and
//                      a lane's 8 consecutive keys of one d are 16 bytes;
// fp32 models use K[s][d] and V[d][s].
struct KvPages {
    const int *tab;  // [rows][ld] block ids, or NULL for the static cache
    int ld;          // entries per row
    int shift;       // log2 of the block size
};

// Stream of position pos of (row b, KV head kvh) and the offset in it.
__device__ __forceinline__ int64_t kv_stream(const KvPages &pg, int b, int kvh, int pos, int Hkv, int &off)
{
    if (pg.tab) {
        off = pos & ((1 << pg.shift) - 1);
        return (int64_t)pg.tab[(int64_t)b * pg.ld + (pos >> pg.shift)] * Hkv + kvh;
    }
    off = pos;
    return (int64_t)b * Hkv + kvh;
}

// Element offsets of (position at offset off of stream st, d) for streams of
// Sb positions.
__host__ __device__ inline int64_t k_offset(int64_t st, int off, int d, int Sb, int hd)
{
    return (st * Sb + off) * hd + d;
}
// fp16 K (head_dim 128): each 32-position block of a stream is stored in the
// operand order of the attention kernels, eight 1 KiB blocks (t, s), t = 0..1
// the 16-key sub-tile, s = 0..3 the 32-wide d chunk: lane r + 16 g of block
// (t, s) holds key 8 (r / 4) + 4 t + r % 4 of the 32 and d = 32 s + 8 g .. +7,
// so every load of a K operand reads 1 KiB contiguously.
__host__ __device__ inline int64_t k16_offset(int64_t st, int off, int d, int Sb, int hd)
{
    const int kk = off & 31, t = (kk >> 2) & 1, r = ((kk >> 3) << 2) | (kk & 3);
    return (st * Sb + (off & ~31)) * hd + ((t * 4 + (d >> 5)) * 64 + r + 16 * ((d >> 3) & 3)) * 8 + (d & 7);
}
__host__ __device__ inline int64_t v16_offset(int64_t st, int off, int d, int Sb, int hd)
{
    return (st * Sb + (off & ~31)) * hd + d * 32 + (off & 31);
}
__host__ __device__ inline int64_t v32_offset(int64_t st, int off, int d, int Sb, int hd)
{
    return (st * hd + d) * Sb + off;
}

// One 16-byte global -> LDS copy per lane (LDS address m0 + 16 * lane).  It
// is issued from inline assembly: with the compiler's own LDS-DMA builtin in
// the loop, its wait-count model stops trusting the in-order completion of
// LDS reads and waits for all of them before the first MFMA of a step.  The
// kernels track these copies themselves with explicit vmcnt waits; m0 is used by
// nothing else in the kernel.
__device__ __forceinline__ void lds_copy16(const void *gsrc, const void *ldst)
{
    const uint32_t l = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)ldst);
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gsrc), "s"(l) : "memory", "m0");
}

// Decode activations of 2 < M <= 32 rows, "fragment-major": the B operand of
// v_mfma_f32_16x16x32_f16 for 16 rows and 32 columns is one contiguous
// 1 KiB block, so a product's activation load is as coalesced as its weight
// load.  Layout [K/32][mh][64 lanes][8] with mh = ceil(M/16) row halves;
// element (m, k) lies in lane (m%16) + 16*((k%32)/8) of block (k/32, m/16).
// Rows m >= M of the last half are never read.
__host__ __device__ inline int64_t xt_offset(int m, int64_t k, int mh)
{
    return (((k >> 5) * mh + (m >> 4)) * 64 + (m & 15) + 16 * ((k & 31) >> 3)) * 8 + (k & 7);
}

// Activation layouts handed between kernels (fp16 models):
//   ACT_ROWS   row-major [M][K] with a row stride;
//   1, 2       the fragment-major decode layout above with that many row halves;
//   ACT_TILED  the weight tile layout applied to activation rows,
//              [ceil(M/16)][K/32][64 lanes][8] (prefill products of >= 1024
//              rows): a stage of the 256 x 256 product loads each 16-row
//              block as one contiguous 1 KiB piece.
enum { ACT_ROWS = 0, ACT_TILED = 3 };
__host__ __device__ inline int64_t act_offset(int m, int64_t k, int64_t K, int64_t ld, int lay)
{
    if (lay == ACT_TILED) return tiled_offset(m, k, K);
    if (lay) return xt_offset(m, k, lay);
    return (int64_t)m * ld + k;
}

// Where activation row m of a forward pass sits (batch row b, position pos):
//  - packed rows of different lengths (varlen prefill): rowmap[m] = {b, pos};
//  - per-row decode positions (T == 1): b = m, pos = pos_rows[m];
//  - otherwise b = m / T and pos = base + m % T, base = *pos_dev or pos_imm.
__device__ __forceinline__ void locate_row(int m, int T, const int *pos_dev, int pos_imm, const int *pos_rows,
                                           const int2 *rowmap, int &b, int &pos)
{
    if (rowmap) {
        const int2 r = rowmap[m];
        b = r.x;
        pos = r.y;
    } else if (pos_rows) {
        b = m;
        pos = pos_rows[m];
    } else {
        b = m / T;
        pos = (pos_dev ? *pos_dev : pos_imm) + m % T;
    }
}

// Packed matrices of one layer, in stored row order.
enum Mat { MAT_QKV = 0, MAT_O = 1, MAT_W13 = 2, MAT_W2 = 3, MAT_HEAD = 4, MAT_EMB = 5 };

// Epilogue kinds applied to the fp32 accumulator of a linear layer.
enum EpKind {
    EP_STORE = 0,   // out[m][n] = round(acc)
    EP_RESID = 1,   // res[m][n] = round(res[m][n] + round(acc))
    EP_LOGITS = 2,  // out_f32[m][n] = round(acc) widened to fp32
    EP_QKV = 3,     // RoPE on q and k, q to out, k/v to the KV cache
    EP_SWIGLU = 4   // g[m][f] = round(round(silu(a)) * b) from interleaved rows
};

// Everything an epilogue needs; unused fields are ignored.
struct Epilogue {
    int kind;
    void *out;            // STORE / RESID / LOGITS / QKV (q) / SWIGLU (g)
    int64_t ldo;          // row stride of out in elements
    // EP_QKV
    void *kcache;         // this layer's K cache (layout above)
    void *vcache;         // this layer's V cache (layout above)
    const float *rope;    // [S][hd/2][2] cos, sin
    const int *pos_dev;   // device position of token 0 (decode) or NULL
    int pos_imm;          // position of token 0 when pos_dev is NULL
    int T;                // tokens per batch row (m = b*T + t)
    const int *pos_rows;  // per-row decode positions, or NULL (locate_row)
    const int2 *rowmap;   // packed varlen rows {b, pos}, or NULL (locate_row)
    int H, Hkv, hd, S;    // S: positions per cache stream (max_seq_len, or the block size when paged)
    KvPages pg;           // block tables of a paged cache (pg.tab NULL: static cache)
    int *pos_advance;     // EP_LOGITS: incremented once after the product (a captured decode step), or NULL
    int out_lay;          // EP_SWIGLU: layout of g (ACT_ROWS with ldo, 1/2 fragment-major, ACT_TILED)
    // split-K decode products: fp32 workspace for the partial sums
    // [splits][M][N] (kSplitMaxFloats floats), or NULL (no split)
    float *part;
};
constexpr int64_t kSplitMaxFloats = 4ll * 32 * 16384;

// ---------------------------------------------------------------------------
// Kernel launchers (each file defines its own); all return hipError_t.
// ---------------------------------------------------------------------------
struct GemmArgs {
    const void *W;     // packed weights (tiled fp16 / row-major fp32)
    const void *X;     // activations [M][K] (row stride ldx), or fragment-major
    int64_t ldx;
    int x_lay;         // layout of X: ACT_ROWS, 1/2 (fragment-major, M <= 32) or ACT_TILED (M >= 1024)
    int M, N, K;
    Epilogue ep;
    const void *norm_w;  // RMSNorm weight applied to the X rows first (only where
                         // skinny_can_normalise(M, K)), or NULL
    float eps;
    // with norm_w: X is the embedding table and row m is the embedding of
    // token gather_tok[b][pos] (b, pos of row m as the epilogue locates it);
    // the raw rows are also stored to gather_out [M][K].  Or NULL.
    const int32_t *gather_tok;
    int64_t gather_ld;
    void *gather_out;
    // residual products of 3..32 fragment-major rows: if not NULL, a split-K
    // form may leave its partial sums in ep.part for the caller's next
    // normalisation launch (launch_rmsnorm_resid) instead of reducing them;
    // *pending is set to the number of splits left there, else 0
    int *pending;
};

// Whether the fp16 product normalises its own input rows for M rows of K.
bool skinny_can_normalise(int M, int K);

hipError_t launch_gen_weights_f16(half_t *dst, int mat, int64_t N, int64_t K, uint64_t seed,
                                  int layer, int H, int Hkv, int hd, int F, bool tiled,
                                  hipStream_t s);
hipError_t launch_gen_weights_f32(float *dst, int mat, int64_t N, int64_t K, uint64_t seed,
                                  int layer, int H, int Hkv, int hd, int F, hipStream_t s);
hipError_t launch_fill_f16(half_t *dst, int64_t n, float v, hipStream_t s);
hipError_t launch_fill_f32(float *dst, int64_t n, float v, hipStream_t s);
hipError_t launch_zero_bytes(void *dst, int64_t bytes, hipStream_t s);
hipError_t launch_read_weights(const void *src, int dtype, int mat, int64_t N, int64_t K,
                               int which, int H, int Hkv, int hd, int F, int64_t first,
                               int64_t count, void *out, hipStream_t s);

// M rows: row m embeds tok[b][pos] with (b, pos) from locate_row.
hipError_t launch_embed(const void *E, const int32_t *tok, int64_t tok_ld, int M, int T,
                        const int *pos_dev, int pos0, const int *pos_rows, const int2 *rowmap, int D,
                        int dtype, void *x, hipStream_t s);
// out[i] = x[idx[i]] for n rows of D elements (es bytes each)
hipError_t launch_gather_rows(const void *x, const int *idx, int n, int D, int es, void *out, hipStream_t s);
// y_lay: layout of y (fp16 only for non-row-major layouts).
hipError_t launch_rmsnorm(const void *x, int64_t ldx, const void *w, int M, int D, float eps,
                          int dtype, void *y, hipStream_t s, int y_lay = ACT_ROWS);
// fp16, M <= 64 rows of x [M][D] (row stride D): first adds the split-K
// partial sums part[S][M][D] of a residual product to x (in split order, with
// the residual epilogue's rounding) and stores x, then normalises as above
hipError_t launch_rmsnorm_resid(const float *part, int S, void *x, const void *w, int M, int D, float eps, void *y,
                                hipStream_t s, int y_lay);

hipError_t launch_gemm_f16(const GemmArgs &a, hipStream_t s);
hipError_t launch_linear_f32(const GemmArgs &a, hipStream_t s);

struct AttnArgs {
    const void *q;         // [B*T][H][hd]
    const void *kcache;    // layout above
    const void *vcache;    // layout above
    void *out;             // [B*T][H][hd]
    int B, T, H, Hkv, hd, S;
    const int *pos_dev;    // decode: device position, else NULL
    int pos_imm;
    int out_lay;           // layout of out as [B*T][H*hd] rows (fp16)
    const int *pos_rows;   // decode with per-row positions (T == 1), or NULL
    const int *cu;         // varlen prefill: row b's queries are packed rows cu[b]..cu[b+1]-1
                           // at positions 0..; T is then the longest row; or NULL
    int Sb;                // positions per cache stream (S, or the block size when paged)
    KvPages pg;            // block tables of a paged cache (pg.tab NULL: static cache)
};
hipError_t launch_attn_decode_f16(const AttnArgs &a, hipStream_t s);
hipError_t launch_attn_prefill_f16(const AttnArgs &a, hipStream_t s);
hipError_t launch_attn_f32(const AttnArgs &a, hipStream_t s);
hipError_t launch_kv_write(const void *k, const void *v, int B, int T, int pos0, int Hkv, int hd,
                           int Sb, const KvPages &pg, int dtype, void *kcache, void *vcache, hipStream_t s);


// Samplers write token column write_col of every row, or with col_rows
// column col_rows[b] + 1 of row b (none when that reaches tok_ld).
hipError_t launch_argmax(const float *logits, int B, int V, int32_t *tok, int64_t tok_ld,
                         int write_col, const int *col_rows, int32_t *out, hipStream_t s);
hipError_t launch_softmax_temp(const float *logits, int B, int V, float temperature,
                               float *probs, hipStream_t s);
hipError_t launch_top_p(const float *probs, int B, int V, float top_p, const float *uniforms,
                        int32_t *tok, int64_t tok_ld, int write_col, const int *col_rows, int32_t *out,
                        hipStream_t s);
// Temperature softmax (from_logits) and top-p in one launch for V <= 32768,
// else the two-launch path through probs_scratch[B][V].
hipError_t launch_sample_top_p(const float *src, bool from_logits, float temperature, int B, int V, float top_p,
                               const float *uniforms, int32_t *tok, int64_t tok_ld, int write_col,
                               const int *col_rows, int32_t *out, float *probs_scratch, hipStream_t s);
// Message of the last failed handle-free call on this thread ("" if none).
const char *static_call_error();
hipError_t launch_set_int(int *dst, int v, hipStream_t s);
// dst[i] += 1 for i < n
hipError_t launch_inc_ints(int *dst, int n, hipStream_t s);
// tok[b][col_rows[b] + 1] = vals[b] for the rows mask selects (all when NULL)
hipError_t launch_set_tokens_rows(int32_t *tok, int64_t tok_ld, int B, const int *col_rows, const int32_t *vals,
                                  const uint8_t *mask, hipStream_t s);
// packed varlen tokens vals[m] -> tok[b][pos] with rowmap[m] = {b, pos}
hipError_t launch_scatter_tokens(int32_t *tok, int64_t tok_ld, int M, const int2 *rowmap, const int32_t *vals,
                                 hipStream_t s);
hipError_t launch_set_tokens(int32_t *tok, int64_t tok_ld, int B, int col, const int32_t *vals,
                             const uint8_t *mask, hipStream_t s);

