// Host side of the library: parameter checks, call-protocol state, device
// memory plan, and the order of kernels for a prefill and a decode step.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <set>
#include <string>
#include <vector>

#include "../../include/llm.h"
#include "common.h"

namespace {

struct Dims {
    int NL, D, H, Hkv, hd, F, V, maxB, S, dtype, es;
    int64_t Nqkv;
};

int64_t ffn_width(const llm_params *p)
{
    // walkthrough section 3.6: int(2 * 4d / 3), optional int(mult * h), round
    // up to multiple_of
    int64_t h = 4 * (int64_t)p->dim;
    h = (int64_t)(2.0 * (double)h / 3.0);
    if (p->ffn_dim_multiplier > 0.0f) h = (int64_t)((double)p->ffn_dim_multiplier * (double)h);
    int64_t mo = p->multiple_of;
    return mo * ((h + mo - 1) / mo);
}

std::string check(const llm_params *p, Dims *d)
{
    if (!p) return "params is NULL";
    if (p->n_layers < 1) return "n_layers must be >= 1";
    if (p->dim < 2 || p->n_heads < 1 || p->dim % p->n_heads) return "dim must be a positive multiple of n_heads";
    int Hkv = p->n_kv_heads > 0 ? p->n_kv_heads : p->n_heads;
    if (Hkv > p->n_heads || p->n_heads % Hkv) return "n_heads must be a multiple of n_kv_heads";
    if (p->vocab_size < 2) return "vocab_size must be >= 2";
    if (p->multiple_of < 1) return "multiple_of must be >= 1";
    if (!(p->norm_eps > 0.f) || !std::isfinite(p->norm_eps)) return "norm_eps must be positive";
    if (!(p->rope_theta > 0.f) || !std::isfinite(p->rope_theta)) return "rope_theta must be positive";
    if (!std::isfinite(p->ffn_dim_multiplier)) return "ffn_dim_multiplier must be finite";
    if (p->max_batch_size < 1 || p->max_batch_size > 4096) return "max_batch_size must be in [1, 4096]";
    if (p->max_seq_len < 1) return "max_seq_len must be >= 1";
    if (p->dtype != LLM_F16 && p->dtype != LLM_F32) return "dtype must be LLM_F16 or LLM_F32";
    int hd = p->dim / p->n_heads;
    if (hd % 2) return "head_dim must be even (RoPE pairs)";
    int64_t F = ffn_width(p);
    if (F < 1 || F > (1 << 24)) return "ffn width out of range";
    if (p->dtype == LLM_F16) {
        if (hd != 128) return "fp16 models need head_dim 128";
        if (p->dim % 64 || p->dim > 8192) return "fp16 models need dim % 64 == 0 and dim <= 8192";
        if (F % 64) return "fp16 models need the ffn width to be a multiple of 64";
        if (p->vocab_size % 16) return "fp16 models need vocab_size % 16 == 0";
        if (p->max_seq_len % 64) return "fp16 models need max_seq_len % 64 == 0";
        if (p->n_heads / Hkv > 16) return "fp16 models need n_heads / n_kv_heads <= 16";
    } else {
        if (p->dim > 4096) return "fp32 models are limited to dim <= 4096";
        if (p->max_seq_len > 8192) return "fp32 models are limited to max_seq_len <= 8192";
    }
    if (p->vocab_size > (1 << 22)) return "vocab_size too large";
    if (d) {
        d->NL = p->n_layers; d->D = p->dim; d->H = p->n_heads; d->Hkv = Hkv; d->hd = hd;
        d->F = (int)F; d->V = p->vocab_size; d->maxB = p->max_batch_size; d->S = p->max_seq_len;
        d->dtype = p->dtype; d->es = p->dtype == LLM_F16 ? 2 : 4;
        d->Nqkv = (int64_t)(p->n_heads + 2 * Hkv) * hd;
    }
    return "";
}

inline int64_t align256(int64_t b) { return (b + 255) & ~(int64_t)255; }

}  // namespace

struct llm {
    llm_params p{};
    Dims d{};
    bool dry = false;
    hipStream_t stream = nullptr;
    bool own_stream = false;
    // weights
    char *emb = nullptr, *wts = nullptr, *norm_w = nullptr;
    std::vector<char *> wqkv, wo, w13, w2;
    char *whead = nullptr;
    // cache and buffers
    char *kv = nullptr;
    int64_t kv_layer_bytes = 0;  // K part then V part
    // paged cache (bs > 0): a pool of kv_blocks blocks of bs positions; row b's
    // positions [bs*i, bs*i + bs) live in block btab[b * bt_ld + i] (-1: none)
    int bs = 0, bshift = 0, kv_blocks = 0, bt_ld = 0;
    std::vector<int> btab;     // host copy, the authority
    std::vector<int> owner;    // [kv_blocks] row holding the block, or -1
    std::set<int> free_ids;    // unheld blocks; allocation takes the lowest
    int *btab_d = nullptr;     // device copy, refreshed before a forward pass
    int *btab_stage = nullptr; // pinned staging buffer of that refresh
    hipEvent_t btab_ev = nullptr;  // the last refresh's read of the staging buffer
    bool btab_dirty = false;
    float kv_util = 0.f;       // memory budget of a pool sized at creation
    float *rope = nullptr;
    int32_t *tok = nullptr;
    float *logits = nullptr, *probs = nullptr, *uni = nullptr;
    int32_t *outtok = nullptr, *stage_i32 = nullptr;
    float *uni_stage = nullptr;    // pinned staging of host uniforms
    hipEvent_t uni_ev = nullptr;   // the last copy out of uni_stage
    uint8_t *stage_mask = nullptr;
    int *pos_dev = nullptr;
    int dev_pos = -1;         // what *pos_dev holds once the queued work has run (-1: unknown)
    int *pos_rows = nullptr;  // [maxB] per-row last written position (rows mode)
    int *cu = nullptr;        // [maxB + 1] varlen row starts, then [maxB] last packed rows
    // activations, sized for ws_rows rows
    char *ws = nullptr;
    int64_t ws_rows = 0;
    char *x = nullptr, *xn = nullptr, *q = nullptr, *o = nullptr, *g = nullptr;
    int2 *rowmap = nullptr;   // varlen prefill: {b, pos} per packed row
    int32_t *vtok = nullptr;  // varlen prefill: packed tokens
    float *part = nullptr;    // split-K partial sums of decode products (kSplitMaxFloats)
    // state.  Uniform mode: every row at last_pos.  Rows mode (after a varlen
    // prefill): row b at row_last[b], its next token column written when
    // row_next[b] is set.
    bool prefilled = false, logits_valid = false, poisoned = false;
    int cur_B = 0, last_pos = -1;
    std::vector<uint8_t> col_written;
    bool rows_mode = false;
    std::vector<int> row_last;
    std::vector<uint8_t> row_next;
    std::string err;
    // decode graphs (uniform positions / per-row positions)
    hipGraphExec_t gexec = nullptr;
    int graph_B = -1;
    hipGraphExec_t gexec_rows = nullptr;
    int graph_rows_B = -1;
    bool use_graph = true;
};

namespace {

int fail(llm_t *h, int code, const std::string &msg)
{
    if (h) {
        h->err = msg;
        if (code == LLM_EDEVICE) h->poisoned = true;
    }
    return code;
}

#define HIPC(h, call)                                                                        \
    do {                                                                                     \
        hipError_t e_ = (call);                                                              \
        if (e_ != hipSuccess)                                                                \
            return fail((h), LLM_EDEVICE, std::string(#call) + ": " + hipGetErrorString(e_)); \
    } while (0)

#define HIPM(h, call)                                                                       \
    do {                                                                                    \
        hipError_t e_ = (call);                                                             \
        if (e_ == hipErrorOutOfMemory) {                                                    \
            (void)hipGetLastError();                                                        \
            return fail((h), LLM_ENOMEM, std::string(#call) + ": out of device memory");    \
        }                                                                                   \
        if (e_ != hipSuccess)                                                               \
            return fail((h), LLM_EDEVICE, std::string(#call) + ": " + hipGetErrorString(e_)); \
    } while (0)

int guard(llm_t *h)
{
    if (!h) return LLM_EINVAL;
    if (h->poisoned) return LLM_EDEVICE;
    return LLM_OK;
}

char *layer_kc(llm_t *h, int l) { return h->kv + (int64_t)l * h->kv_layer_bytes; }
char *layer_vc(llm_t *h, int l) { return h->kv + (int64_t)l * h->kv_layer_bytes + h->kv_layer_bytes / 2; }

// Activation workspace for `rows` token rows (grows, never shrinks).
int ensure_ws(llm_t *h, int64_t rows)
{
    rows = rows < 32 ? 32 : (rows + 15) / 16 * 16;  // laid-out activations span whole 16-row blocks
    if (rows <= h->ws_rows) return LLM_OK;
    const Dims &d = h->d;
    int64_t bx = align256(rows * d.D * d.es), bq = align256(rows * (int64_t)d.H * d.hd * d.es),
            bg = align256(rows * (int64_t)d.F * d.es);
    if (h->ws) {
        HIPC(h, hipStreamSynchronize(h->stream));
        HIPC(h, hipFree(h->ws));
        h->ws = nullptr;
        h->ws_rows = 0;
    }
    void *p = nullptr;
    const int64_t br = align256(rows * (int64_t)sizeof(int2)), bt = align256(rows * 4),
                  bp = align256(kSplitMaxFloats * (int64_t)sizeof(float));
    HIPM(h, hipMalloc(&p, 2 * bx + 2 * bq + bg + br + bt + bp));
    h->ws = (char *)p;
    h->x = h->ws;
    h->xn = h->x + bx;
    h->q = h->xn + bx;
    h->o = h->q + bq;
    h->g = h->o + bq;
    h->rowmap = (int2 *)(h->g + bg);
    h->vtok = (int32_t *)((char *)h->rowmap + br);
    h->part = (float *)((char *)h->vtok + bt);
    h->ws_rows = rows;
    // the captured decode graphs hold the old addresses
    if (h->gexec) {
        (void)hipGraphExecDestroy(h->gexec);
        h->gexec = nullptr;
        h->graph_B = -1;
    }
    if (h->gexec_rows) {
        (void)hipGraphExecDestroy(h->gexec_rows);
        h->gexec_rows = nullptr;
        h->graph_rows_B = -1;
    }
    return LLM_OK;
}

// ---------------------------------------------------------------------------
// Paged KV cache (nano-vllm notes, allocate_kv_cache and the block tables).
// ---------------------------------------------------------------------------
// Bytes of one block: K and V of bs positions of every KV head of every layer.
int64_t block_bytes(const Dims &d, int bs) { return 2 * (int64_t)d.NL * bs * d.Hkv * d.hd * d.es; }

std::string check_paging(const Dims &d, const llm_paging *pg, bool dry)
{
    if (!pg) return "paging is NULL";
    const int bs = pg->block_size;
    if (bs < 32 || bs > (1 << 16) || (bs & (bs - 1))) return "block_size must be a power of two in [32, 65536]";
    const int64_t cap = (int64_t)d.maxB * ((d.S + bs - 1) / bs);
    if (pg->num_blocks < 0 || pg->num_blocks > cap)
        return "num_blocks must be in [0, max_batch_size * ceil(max_seq_len / block_size)]";
    if (pg->num_blocks == 0) {
        if (dry) return "a dry handle needs num_blocks > 0";
        if (!(pg->gpu_memory_utilization > 0.f && pg->gpu_memory_utilization <= 1.f))
            return "gpu_memory_utilization must be in (0, 1]";
    }
    return "";
}

// Host bookkeeping of a pool of n blocks, every block free.
void init_pages(llm_t *h, int n)
{
    h->kv_blocks = n;
    h->btab.assign((size_t)h->d.maxB * h->bt_ld, -1);
    h->owner.assign(n, -1);
    h->free_ids.clear();
    for (int i = 0; i < n; i++) h->free_ids.insert(h->free_ids.end(), i);
    h->btab_dirty = true;
}

// The pool: num_blocks blocks, or with num_blocks == 0 as many as the
// budget allows: total * utilisation - memory in use once everything else,
// including the activation workspace of the largest pass, is allocated
// (the transient peak of a forward pass is reserved before measuring).
// More blocks than every row at max_seq_len could hold are never taken.
int alloc_pool(llm_t *h)
{
    const Dims &d = h->d;
    const int64_t per_block = block_bytes(d, h->bs), cap = (int64_t)d.maxB * h->bt_ld;
    int64_t n = h->kv_blocks;
    if (n == 0) {
        int rc = ensure_ws(h, (int64_t)d.maxB * d.S);
        if (rc) return rc;
        size_t fr = 0, tot = 0;
        HIPC(h, hipMemGetInfo(&fr, &tot));
        const double budget = (double)tot * h->kv_util - (double)(tot - fr);
        n = budget > 0 ? (int64_t)(budget / (double)per_block) : 0;
        if (n < 1) return fail(h, LLM_ENOMEM, "the memory budget leaves no room for one KV block");
        n = std::min(n, cap);
    }
    void *p = nullptr;
    h->kv_layer_bytes = per_block / d.NL * n;
    HIPM(h, hipMalloc(&p, h->kv_layer_bytes * d.NL));
    h->kv = (char *)p;
    HIPC(h, launch_zero_bytes(h->kv, h->kv_layer_bytes * d.NL, h->stream));
    init_pages(h, (int)n);  // sizes the host tables
    const size_t tb = h->btab.size() * sizeof(int);
    HIPM(h, hipMalloc(&p, tb));
    h->btab_d = (int *)p;
    HIPM(h, hipHostMalloc(&p, tb, hipHostMallocDefault));
    h->btab_stage = (int *)p;
    HIPC(h, hipEventCreateWithFlags(&h->btab_ev, hipEventDisableTiming));
    return LLM_OK;
}

// Give every row b < B blocks for positions [0, end[b]) after checking that
// the positions [0, read_end[b]) it reads are held; with release_rest the
// blocks of rows >= B are returned to the pool first (a prefill from position
// 0 ends those rows).  All or nothing: on error no table changes.
int kv_reserve(llm_t *h, int B, const std::vector<int> &read_end, const std::vector<int> &end, bool release_rest)
{
    if (!h->bs) return LLM_OK;
    const int ld = h->bt_ld;
    int64_t avail = (int64_t)h->free_ids.size(), need = 0;
    if (release_rest)
        for (size_t i = (size_t)B * ld; i < h->btab.size(); i++) avail += h->btab[i] >= 0;
    for (int b = 0; b < B; b++) {
        const int nr = (read_end[b] + h->bs - 1) >> h->bshift, ne = (end[b] + h->bs - 1) >> h->bshift;
        for (int i = 0; i < nr; i++)
            if (h->btab[(size_t)b * ld + i] < 0)
                return fail(h, LLM_ESTATE, "row " + std::to_string(b) + " holds no block for cached positions it reads");
        for (int i = nr; i < ne; i++) need += h->btab[(size_t)b * ld + i] < 0;
    }
    if (need > avail)
        return fail(h, LLM_ENOMEM, "KV block pool exhausted: " + std::to_string(need) + " blocks needed, " +
                                       std::to_string(avail) + " free");
    if (release_rest)
        for (size_t i = (size_t)B * ld; i < h->btab.size(); i++)
            if (h->btab[i] >= 0) {
                h->owner[h->btab[i]] = -1;
                h->free_ids.insert(h->btab[i]);
                h->btab[i] = -1;
                h->btab_dirty = true;
            }
    for (int b = 0; b < B; b++) {
        const int ne = (end[b] + h->bs - 1) >> h->bshift;
        for (int i = 0; i < ne; i++) {
            int &e = h->btab[(size_t)b * ld + i];
            if (e >= 0) continue;
            e = *h->free_ids.begin();
            h->free_ids.erase(h->free_ids.begin());
            h->owner[e] = b;
            h->btab_dirty = true;
        }
    }
    return LLM_OK;
}

// Same positions for every row b < B.
int kv_reserve_uniform(llm_t *h, int B, int read_end, int end, bool release_rest)
{
    return kv_reserve(h, B, std::vector<int>(B, read_end), std::vector<int>(B, end), release_rest);
}

// Bring the device block tables up to date (outside any graph capture).
int kv_upload(llm_t *h)
{
    if (!h->bs || h->dry || !h->btab_dirty) return LLM_OK;
    HIPC(h, hipEventSynchronize(h->btab_ev));  // the previous copy has read the staging buffer
    const size_t tb = h->btab.size() * sizeof(int);
    memcpy(h->btab_stage, h->btab.data(), tb);
    HIPC(h, hipMemcpyAsync(h->btab_d, h->btab_stage, tb, hipMemcpyHostToDevice, h->stream));
    HIPC(h, hipEventRecord(h->btab_ev, h->stream));
    h->btab_dirty = false;
    return LLM_OK;
}

KvPages kv_pages(const llm_t *h)
{
    KvPages pg{};
    if (h->bs) {
        pg.tab = h->btab_d;
        pg.ld = h->bt_ld;
        pg.shift = h->bshift;
    }
    return pg;
}

// Positions per cache stream: the block size of a paged cache, else max_seq_len.
int stream_len(const llm_t *h) { return h->bs ? h->bs : h->d.S; }

int64_t mat_rows(const Dims &d, int mat)
{
    switch (mat) {
    case MAT_QKV: return d.Nqkv;
    case MAT_O: return d.D;
    case MAT_W13: return 2 * (int64_t)d.F;
    case MAT_W2: return d.D;
    default: return d.V;
    }
}

int64_t mat_cols(const Dims &d, int mat)
{
    switch (mat) {
    case MAT_O: return (int64_t)d.H * d.hd;
    case MAT_W2: return d.F;
    default: return d.D;
    }
}

const char *mat_ptr(llm_t *h, int layer, int mat)
{
    switch (mat) {
    case MAT_QKV: return h->wqkv[layer];
    case MAT_O: return h->wo[layer];
    case MAT_W13: return h->w13[layer];
    case MAT_W2: return h->w2[layer];
    case MAT_HEAD: return h->whead;
    default: return h->emb;
    }
}

hipError_t run_linear(llm_t *h, int layer, int mat, const void *X, int64_t ldx, int M,
                      const Epilogue &ep, const void *norm_w = nullptr, int x_lay = ACT_ROWS,
                      const int32_t *gather_tok = nullptr, int *pending = nullptr)
{
    GemmArgs a{};
    a.pending = pending;
    a.gather_tok = gather_tok;
    a.gather_ld = h->d.S;
    a.gather_out = h->x;
    a.W = mat_ptr(h, layer, mat);
    a.X = X;
    a.ldx = ldx;
    a.x_lay = x_lay;
    a.M = M;
    a.N = (int)mat_rows(h->d, mat);
    a.K = (int)mat_cols(h->d, mat);
    a.ep = ep;
    a.norm_w = norm_w;
    a.eps = h->p.norm_eps;
    return h->d.dtype == LLM_F16 ? launch_gemm_f16(a, h->stream) : launch_linear_f32(a, h->stream);
}

// RMSNorm followed by a product: folded into the product (rows staged and
// normalised in LDS) for one or two fp16 rows, else a normalisation kernel
// writing xn and the product on xn.
bool fuse_norm(const llm_t *h, int M) { return h->d.dtype == LLM_F16 && skinny_can_normalise(M, h->d.D); }

// One forward pass: B batch rows, M activation rows.
//  - uniform prefill: T tokens per row at pos0.. (M = B*T);
//  - decode (T = 1): position from pos_dev (all rows) or pos_rows (per row);
//  - varlen prefill: rows of different lengths packed (M = their sum),
//    rowmap gives {b, pos} per packed row, cu the row starts, last_rows the
//    packed index of each row's last token, Tmax the longest row.
struct Pass {
    int B = 0, T = 1, M = 0;
    const int *pos_dev = nullptr;
    int pos0 = 0;
    const int *pos_rows = nullptr;
    const int2 *rowmap = nullptr;
    const int *cu = nullptr, *last_rows = nullptr;
    int Tmax = 0;
    bool advance = false;  // the head's product moves *pos_dev on by one (captured decode steps)
    bool x_given = false;  // the residual rows are already in x: layer 0 does not gather embeddings
    bool decode() const { return pos_dev || pos_rows; }
};

Pass uniform_pass(int B, int T, const int *pos_dev, int pos0 = 0)
{
    Pass p;
    p.B = B;
    p.T = T;
    p.M = B * T;
    p.pos_dev = pos_dev;
    p.pos0 = pos0;
    return p;
}

// Layout of the activations a forward pass hands to its layer products
// (normalised rows, attention output, SwiGLU output): decode steps of 3..32
// fp16 rows use the fragment-major layout (row halves of 16), fp16 prefills
// of >= 1024 rows the weight tile layout; everything else is row-major.
// Row-major always for the output head, whose M is the batch.
constexpr int kTiledMinRows = 1024;  // the 256 x 256 product takes M >= 1024

int act_layout(const llm_t *h, const Pass &ps)
{
    if (h->d.dtype != LLM_F16) return ACT_ROWS;
    if (ps.decode()) return ps.B > 2 && ps.B <= 32 ? (ps.B + 15) / 16 : ACT_ROWS;
    if (ps.M >= kTiledMinRows) return ACT_TILED;
    return ACT_ROWS;
}

int head_layout(int lay) { return lay == ACT_TILED ? ACT_ROWS : lay; }

Epilogue make_ep(int kind, void *out, int64_t ldo)
{
    Epilogue e{};
    e.kind = kind;
    e.out = out;
    e.ldo = ldo;
    e.T = 1;
    return e;
}

// Optional per-launch timing: events recorded around every kernel of a
// forward pass, attributed to a kernel class.
struct Prof {
    std::vector<hipEvent_t> ev;  // pairs
    std::vector<int> cls;
    size_t used = 0;
};

enum ProfClass {
    PC_EMBED = 0, PC_NORM = 1, PC_QKV = 2, PC_ATTN = 3, PC_O = 4, PC_W13 = 5, PC_W2 = 6, PC_HEAD = 7,
    PC_N = 9  // the last slot holds the first-to-last event time
};

hipError_t prof_mark(Prof *pf, int cls, hipStream_t s)
{
    if (!pf) return hipSuccess;
    if (pf->used + 2 > pf->ev.size()) {
        for (int i = 0; i < 64; i++) {
            hipEvent_t e;
            hipError_t r = hipEventCreate(&e);
            if (r != hipSuccess) return r;
            pf->ev.push_back(e);
        }
    }
    pf->cls.resize(pf->used / 2 + 1);
    pf->cls[pf->used / 2] = cls;
    return hipEventRecord(pf->ev[pf->used++], s);
}

hipError_t prof_end(Prof *pf, hipStream_t s)
{
    if (!pf) return hipSuccess;
    return hipEventRecord(pf->ev[pf->used++], s);
}

// One weight product of the forward pass with its epilogue: layer l's
// wq|wk|wv (RoPE and the KV-cache write), wo and w2 (residual add), w1|w3
// (SwiGLU), or the output head on the last position of each row (fp32
// logits).  With `fused` the RMSNorm in front of wq|wk|wv, w1|w3 and the
// head runs inside the product on x; otherwise the product reads xn.
// The row-major input of the output head: the last position of each row
// (uniform rows: every T-th row of x; varlen: gathered into q by forward).
const char *head_rows(llm_t *h, const Pass &ps, int64_t *ld)
{
    if (ps.rowmap) {
        *ld = h->d.D;
        return h->q;
    }
    *ld = (int64_t)ps.T * h->d.D;
    return h->x + (int64_t)(ps.T - 1) * h->d.D * h->d.es;
}

// pending (wo, w2): see GemmArgs::pending; NULL to have the product reduce
// any split itself
hipError_t product(llm_t *h, int l, int mat, const Pass &ps, bool fused, int *pending = nullptr)
{
    const Dims &d = h->d;
    const int M = ps.M;
    const int64_t qd = (int64_t)d.H * d.hd;
    const int lay = act_layout(h, ps);
    switch (mat) {
    case MAT_QKV: {
        Epilogue eq = make_ep(EP_QKV, h->q, qd);
        eq.kcache = layer_kc(h, l);
        eq.vcache = layer_vc(h, l);
        eq.rope = h->rope;
        eq.pos_dev = ps.pos_dev;
        eq.pos_imm = ps.pos0;
        eq.pos_rows = ps.pos_rows;
        eq.rowmap = ps.rowmap;
        eq.T = ps.T;
        eq.H = d.H; eq.Hkv = d.Hkv; eq.hd = d.hd; eq.S = stream_len(h);
        eq.pg = kv_pages(h);
        eq.part = h->part;  // 17..32 decode rows may split K
        const char *nw = h->norm_w + (int64_t)(2 * l) * d.D * d.es;
        // fused, layer 0: the product gathers the embedding rows itself and
        // stores them into x (no embedding launch)
        if (fused && l == 0 && !ps.x_given) return run_linear(h, l, MAT_QKV, h->emb, d.D, M, eq, nw, ACT_ROWS, h->tok);
        return fused ? run_linear(h, l, MAT_QKV, h->x, d.D, M, eq, nw)
                     : run_linear(h, l, MAT_QKV, h->xn, d.D, M, eq, nullptr, lay);
    }
    case MAT_O: {
        Epilogue er = make_ep(EP_RESID, h->x, d.D);
        er.part = h->part;
        return run_linear(h, l, MAT_O, h->o, qd, M, er, nullptr, lay, nullptr, pending);
    }
    case MAT_W13: {
        const char *nw = h->norm_w + (int64_t)(2 * l + 1) * d.D * d.es;
        Epilogue eg = make_ep(EP_SWIGLU, h->g, d.F);
        eg.out_lay = lay;
        return fused ? run_linear(h, l, MAT_W13, h->x, d.D, M, eg, nw)
                     : run_linear(h, l, MAT_W13, h->xn, d.D, M, eg, nullptr, lay);
    }
    case MAT_W2: {
        // a long product of 17..32 decode rows may split K (partials in part)
        Epilogue er = make_ep(EP_RESID, h->x, d.D);
        er.part = h->part;
        return run_linear(h, l, MAT_W2, h->g, d.F, M, er, nullptr, lay, nullptr, pending);
    }
    default: {
        const char *nw = h->norm_w + (int64_t)(2 * d.NL) * d.D * d.es;
        int64_t ld = 0;
        const char *xl = head_rows(h, ps, &ld);
        Epilogue el = make_ep(EP_LOGITS, h->logits, d.V);
        el.pos_advance = ps.advance ? h->pos_dev : nullptr;
        return fused ? run_linear(h, 0, MAT_HEAD, xl, ld, ps.B, el, nw)
                     : run_linear(h, 0, MAT_HEAD, h->xn, d.D, ps.B, el, nullptr, head_layout(lay));
    }
    }
}

// State one pass carries from layer to layer: whether RMSNorm runs inside
// the products, the activation layout, and the split count of split-K
// partial sums the last residual product left in h->part for the next
// normalisation launch to add to x (0: none).
struct LayerRun {
    bool fused = false;
    int lay = ACT_ROWS;
    int pend = 0;
};

// The normalisation in front of a product (non-fused forms): adds the
// pending split-K partials to x first when the last residual product handed
// them over, then normalises x into xn.
hipError_t norm_launch(llm_t *h, LayerRun &lr, const void *nw, int rows)
{
    const Dims &d = h->d;
    if (lr.pend) {
        const int sp = lr.pend;
        lr.pend = 0;
        return launch_rmsnorm_resid(h->part, sp, h->x, nw, rows, d.D, h->p.norm_eps, h->xn, h->stream, lr.lay);
    }
    return launch_rmsnorm(h->x, d.D, nw, rows, d.D, h->p.norm_eps, d.dtype, h->xn, h->stream, lr.lay);
}

// TransformerBlock l (walkthrough section 3.7) of the pass ps on the residual
// rows in x: h = x + wo(attention(RoPE(wq|wk|wv(attention_norm(x))))), then
// out = h + w2(silu(w1 ffn_norm(h)) * w3 ffn_norm(h)).  With defer_w2 the
// w2 product may leave split-K partials for the next normalisation launch
// (lr.pend); wo may always do so, the ffn normalisation adds them.
hipError_t layer_pass(llm_t *h, const Pass &ps, int l, LayerRun &lr, bool defer_w2, Prof *pf)
{
    const Dims &d = h->d;
    const int M = ps.M, B = ps.B;
    hipStream_t s = h->stream;
    hipError_t e;
    int *defer = lr.fused ? nullptr : &lr.pend;
    const char *nw_attn = h->norm_w + (int64_t)(2 * l) * d.D * d.es;
    const char *nw_ffn = h->norm_w + (int64_t)(2 * l + 1) * d.D * d.es;
#define TRY_RAW(x)                    \
    do {                              \
        if ((e = (x)) != hipSuccess) \
            return e;                 \
    } while (0)
#define TRYC(cls, x)                       \
    do {                                   \
        TRY_RAW(prof_mark(pf, (cls), s)); \
        TRY_RAW(x);                        \
        TRY_RAW(prof_end(pf, s));          \
    } while (0)
    // attention_norm -> wq|wk|wv with RoPE and the KV-cache write
    if (!lr.fused) TRYC(PC_NORM, norm_launch(h, lr, nw_attn, M));
    TRYC(PC_QKV, product(h, l, MAT_QKV, ps, lr.fused));
    // attention over the cache
    AttnArgs aa{};
    aa.q = h->q; aa.kcache = layer_kc(h, l); aa.vcache = layer_vc(h, l); aa.out = h->o;
    aa.B = B; aa.T = ps.rowmap ? ps.Tmax : ps.T; aa.H = d.H; aa.Hkv = d.Hkv; aa.hd = d.hd; aa.S = d.S;
    aa.Sb = stream_len(h);
    aa.pg = kv_pages(h);
    aa.pos_dev = ps.pos_dev; aa.pos_imm = ps.pos0;
    aa.pos_rows = ps.pos_rows;
    aa.cu = ps.cu;
    aa.out_lay = lr.lay;
    if (d.dtype == LLM_F32) TRYC(PC_ATTN, launch_attn_f32(aa, s));
    else if (ps.decode()) TRYC(PC_ATTN, launch_attn_decode_f16(aa, s));
    else TRYC(PC_ATTN, launch_attn_prefill_f16(aa, s));
    // wo + residual
    TRYC(PC_O, product(h, l, MAT_O, ps, lr.fused, defer));
    // ffn_norm -> w1|w3 with SwiGLU -> w2 + residual
    if (!lr.fused) TRYC(PC_NORM, norm_launch(h, lr, nw_ffn, M));
    TRYC(PC_W13, product(h, l, MAT_W13, ps, lr.fused));
    TRYC(PC_W2, product(h, l, MAT_W2, ps, lr.fused, defer_w2 ? defer : nullptr));
#undef TRYC
#undef TRY_RAW
    return hipSuccess;
}

// The forward pass (walkthrough sections 2, 3.5-3.8) described by ps.
// Decode positions come from device memory so that the launch sequence can
// be captured once and replayed.
hipError_t forward(llm_t *h, const Pass &ps, Prof *pf = nullptr)
{
    const Dims &d = h->d;
    const int M = ps.M, B = ps.B;
    hipStream_t s = h->stream;
    hipError_t e;
#define TRY_RAW(x)                    \
    do {                              \
        if ((e = (x)) != hipSuccess) \
            return e;                 \
    } while (0)
#define TRYC(cls, x)                       \
    do {                                   \
        TRY_RAW(prof_mark(pf, (cls), s)); \
        TRY_RAW(x);                        \
        TRY_RAW(prof_end(pf, s));          \
    } while (0)
    const bool fused = fuse_norm(h, M);
    if (!fused)  // else layer 0's wq|wk|wv product gathers the embedding rows
        TRYC(PC_EMBED, launch_embed(h->emb, h->tok, d.S, M, ps.T, ps.pos_dev, ps.pos0, ps.pos_rows, ps.rowmap, d.D,
                                    d.dtype, h->x, s));
    LayerRun lr;
    lr.fused = fused;
    lr.lay = act_layout(h, ps);
    for (int l = 0; l < d.NL; l++) TRY_RAW(layer_pass(h, ps, l, lr, l + 1 < d.NL, pf));
    // final norm on the last position of each row, output head, fp32 logits
    if (ps.rowmap) TRYC(PC_HEAD, launch_gather_rows(h->x, ps.last_rows, B, d.D, d.es, h->q, s));
    const bool fused_head = fuse_norm(h, B);
    if (!fused_head) {
        const char *nw_final = h->norm_w + (int64_t)(2 * d.NL) * d.D * d.es;
        int64_t ld = 0;
        const char *xl = head_rows(h, ps, &ld);
        TRYC(PC_NORM, launch_rmsnorm(xl, ld, nw_final, B, d.D, h->p.norm_eps, d.dtype, h->xn, s, head_layout(lr.lay)));
    }
    TRYC(PC_HEAD, product(h, 0, MAT_HEAD, ps, fused_head));
#undef TRYC
#undef TRY_RAW
    return hipSuccess;
}

void rope_table_host(int hd, int S, float base, std::vector<float> &t)
{
    // walkthrough section 3.3: theta_i = base^(-2i/d); angle = m * theta_i in
    // fp32; cos and sin of the fp32 angle rounded to fp32.
    const int half = hd / 2;
    t.assign((size_t)S * half * 2, 0.f);
    for (int i = 0; i < half; i++) {
        float th = (float)(1.0 / std::pow((double)base, (double)(2 * i) / (double)hd));
        for (int m = 0; m < S; m++) {
            float ang = (float)m * th;
            t[((size_t)m * half + i) * 2 + 0] = (float)std::cos((double)ang);
            t[((size_t)m * half + i) * 2 + 1] = (float)std::sin((double)ang);
        }
    }
}

int build_weights(llm_t *h, uint64_t seed)
{
    const Dims &d = h->d;
    hipStream_t s = h->stream;
    const int mats[4] = {MAT_QKV, MAT_O, MAT_W13, MAT_W2};
    for (int l = 0; l < d.NL; l++) {
        char *ptrs[4] = {h->wqkv[l], h->wo[l], h->w13[l], h->w2[l]};
        for (int i = 0; i < 4; i++) {
            int64_t N = mat_rows(d, mats[i]), K = mat_cols(d, mats[i]);
            if (d.dtype == LLM_F16)
                HIPC(h, launch_gen_weights_f16((half_t *)ptrs[i], mats[i], N, K, seed, l, d.H, d.Hkv,
                                               d.hd, d.F, true, s));
            else
                HIPC(h, launch_gen_weights_f32((float *)ptrs[i], mats[i], N, K, seed, l, d.H, d.Hkv,
                                               d.hd, d.F, s));
        }
    }
    if (d.dtype == LLM_F16) {
        HIPC(h, launch_gen_weights_f16((half_t *)h->whead, MAT_HEAD, d.V, d.D, seed, 0, d.H, d.Hkv,
                                       d.hd, d.F, true, s));
        HIPC(h, launch_gen_weights_f16((half_t *)h->emb, MAT_EMB, d.V, d.D, seed, 0, d.H, d.Hkv, d.hd,
                                       d.F, false, s));
        HIPC(h, launch_fill_f16((half_t *)h->norm_w, (int64_t)(2 * d.NL + 1) * d.D, 1.0f, s));
    } else {
        HIPC(h, launch_gen_weights_f32((float *)h->whead, MAT_HEAD, d.V, d.D, seed, 0, d.H, d.Hkv,
                                       d.hd, d.F, s));
        HIPC(h, launch_gen_weights_f32((float *)h->emb, MAT_EMB, d.V, d.D, seed, 0, d.H, d.Hkv, d.hd,
                                       d.F, s));
        HIPC(h, launch_fill_f32((float *)h->norm_w, (int64_t)(2 * d.NL + 1) * d.D, 1.0f, s));
    }
    return LLM_OK;
}

int create_impl(llm_t *h, uint64_t seed)
{
    const Dims &d = h->d;
    // weights: every layer matrix and the head in one allocation
    const int mats[4] = {MAT_QKV, MAT_O, MAT_W13, MAT_W2};
    int64_t per_layer = 0, offs[4];
    for (int i = 0; i < 4; i++) {
        offs[i] = per_layer;
        per_layer += align256(mat_rows(d, mats[i]) * mat_cols(d, mats[i]) * d.es);
    }
    int64_t head_bytes = align256((int64_t)d.V * d.D * d.es);
    void *p = nullptr;
    HIPM(h, hipMalloc(&p, per_layer * d.NL + head_bytes));
    h->wts = (char *)p;
    h->wqkv.resize(d.NL); h->wo.resize(d.NL); h->w13.resize(d.NL); h->w2.resize(d.NL);
    for (int l = 0; l < d.NL; l++) {
        char *b = h->wts + (int64_t)l * per_layer;
        h->wqkv[l] = b + offs[0]; h->wo[l] = b + offs[1]; h->w13[l] = b + offs[2]; h->w2[l] = b + offs[3];
    }
    h->whead = h->wts + per_layer * d.NL;
    HIPM(h, hipMalloc(&p, align256((int64_t)d.V * d.D * d.es)));
    h->emb = (char *)p;
    HIPM(h, hipMalloc(&p, align256((int64_t)(2 * d.NL + 1) * d.D * d.es)));
    h->norm_w = (char *)p;
    // static KV cache (walkthrough section 3.1), zeroed; a paged pool is
    // allocated last, from what the rest leaves
    if (!h->bs) {
        h->kv_layer_bytes = 2 * (int64_t)d.maxB * d.Hkv * d.S * d.hd * d.es;
        HIPM(h, hipMalloc(&p, h->kv_layer_bytes * d.NL));
        h->kv = (char *)p;
        HIPC(h, launch_zero_bytes(h->kv, h->kv_layer_bytes * d.NL, h->stream));
    }
    // RoPE table
    std::vector<float> rt;
    rope_table_host(d.hd, d.S, h->p.rope_theta, rt);
    HIPM(h, hipMalloc(&p, rt.size() * sizeof(float)));
    h->rope = (float *)p;
    HIPC(h, hipMemcpyAsync(h->rope, rt.data(), rt.size() * sizeof(float), hipMemcpyHostToDevice, h->stream));
    // token buffer, logits, sampler and attention scratch
    HIPM(h, hipMalloc(&p, (int64_t)d.maxB * d.S * sizeof(int32_t)));
    h->tok = (int32_t *)p;
    HIPC(h, launch_zero_bytes(h->tok, (int64_t)d.maxB * d.S * sizeof(int32_t), h->stream));
    HIPM(h, hipMalloc(&p, (int64_t)d.maxB * d.V * sizeof(float)));
    h->logits = (float *)p;
    HIPM(h, hipMalloc(&p, (int64_t)d.maxB * d.V * sizeof(float)));
    h->probs = (float *)p;
    HIPM(h, hipMalloc(&p, 256 + (int64_t)d.maxB * (sizeof(float) + 5 * sizeof(int32_t) + 1) + 16));
    h->pos_dev = (int *)p;
    h->uni = (float *)((char *)p + 64);
    h->outtok = (int32_t *)(h->uni + d.maxB);
    h->stage_i32 = h->outtok + d.maxB;
    h->pos_rows = h->stage_i32 + d.maxB;
    h->cu = h->pos_rows + d.maxB;  // maxB + 1 starts, then maxB last rows
    h->stage_mask = (uint8_t *)(h->cu + 2 * d.maxB + 1);
    HIPM(h, hipHostMalloc(&p, (size_t)d.maxB * sizeof(float), hipHostMallocDefault));
    h->uni_stage = (float *)p;
    HIPC(h, hipEventCreateWithFlags(&h->uni_ev, hipEventDisableTiming));
    int rc = ensure_ws(h, d.maxB);
    if (rc) return rc;
    rc = build_weights(h, seed);
    if (rc) return rc;
    if (h->bs && (rc = alloc_pool(h))) return rc;
    HIPC(h, hipStreamSynchronize(h->stream));
    return LLM_OK;
}

void release(llm_t *h)
{
    if (h->gexec) (void)hipGraphExecDestroy(h->gexec);
    if (h->gexec_rows) (void)hipGraphExecDestroy(h->gexec_rows);
    void *bufs[] = {h->wts, h->emb, h->norm_w, h->kv, h->rope, h->tok, h->logits, h->probs,
                    h->pos_dev, h->ws, h->btab_d};
    for (void *b : bufs)
        if (b) (void)hipFree(b);
    if (h->btab_stage) (void)hipHostFree(h->btab_stage);
    if (h->uni_stage) (void)hipHostFree(h->uni_stage);
    if (h->uni_ev) (void)hipEventDestroy(h->uni_ev);
    if (h->btab_ev) (void)hipEventDestroy(h->btab_ev);
    if (h->own_stream && h->stream) (void)hipStreamDestroy(h->stream);
}

bool tokens_ok(const int32_t *t, int64_t n, int V)
{
    for (int64_t i = 0; i < n; i++)
        if (t[i] < 0 || t[i] >= V) return false;
    return true;
}

int after_forward(llm_t *h, hipError_t e)
{
    if (e != hipSuccess) return fail(h, LLM_EDEVICE, std::string("kernel launch: ") + hipGetErrorString(e));
    return LLM_OK;
}

int prefill_common(llm_t *h, int B, int T, int start = 0)
{
    if (!h->dry) {
        int rc = ensure_ws(h, (int64_t)B * T);
        if (rc) return rc;
        if ((rc = kv_upload(h))) return rc;
        hipError_t e = forward(h, uniform_pass(B, T, nullptr, start));
        rc = after_forward(h, e);
        if (rc) return rc;
    }
    h->prefilled = true;
    h->logits_valid = true;
    h->rows_mode = false;
    h->cur_B = B;
    h->last_pos = start + T - 1;
    if (start == 0) std::fill(h->col_written.begin(), h->col_written.end(), 0);
    std::fill(h->col_written.begin() + start, h->col_written.begin() + start + T, 1);
    return LLM_OK;
}

int check_prefill_args(llm_t *h, int B, int T, int start = 0)
{
    if (B < 1 || B > h->d.maxB) return fail(h, LLM_EINVAL, "B must be in [1, max_batch_size]");
    if (start < 0) return fail(h, LLM_EINVAL, "start_pos must be >= 0");
    if (T < 1 || (int64_t)start + T > h->d.S) return fail(h, LLM_EINVAL, "need 1 <= T and start_pos + T <= max_seq_len");
    if (start > 0) {
        if (!h->prefilled) return fail(h, LLM_ESTATE, "prefill at an offset needs the cache prefix of an earlier prefill");
        if (h->rows_mode) return fail(h, LLM_ESTATE, "prefill at an offset needs rows at one position (not after a varlen prefill)");
        if (B != h->cur_B) return fail(h, LLM_ESTATE, "prefill at an offset must keep the batch of the cache prefix");
        if (start > h->last_pos + 1) return fail(h, LLM_ESTATE, "start_pos skips positions whose KV is not written");
    }
    return LLM_OK;
}

int sample_check(llm_t *h, float temperature, float top_p, bool have_u)
{
    if (!h->logits_valid) return fail(h, LLM_ESTATE, "no logits: run llm_prefill or llm_decode first");
    if (!std::isfinite(temperature)) return fail(h, LLM_EINVAL, "temperature must be finite");
    if (temperature > 0.f) {
        if (!(top_p > 0.f && top_p <= 1.f)) return fail(h, LLM_EINVAL, "top_p must be in (0, 1]");
        if (!have_u) return fail(h, LLM_EINVAL, "uniforms are required when temperature > 0");
    }
    return LLM_OK;
}

int sample_common(llm_t *h, float temperature, float top_p, const float *uniforms_d, bool have_u,
                  int32_t *out_d)
{
    const Dims &d = h->d;
    int rc0 = sample_check(h, temperature, top_p, have_u);
    if (rc0) return rc0;
    // uniform rows write column last_pos + 1; rows mode column row_last[b] + 1
    const int col = h->last_pos + 1 < d.S ? h->last_pos + 1 : -1;
    const int *col_rows = h->rows_mode ? h->pos_rows : nullptr;
    if (!h->dry) {
        hipError_t e;
        if (temperature <= 0.f) {
            e = launch_argmax(h->logits, h->cur_B, d.V, h->tok, d.S, col, col_rows, out_d, h->stream);
        } else {
            e = launch_sample_top_p(h->logits, true, temperature, h->cur_B, d.V, top_p, uniforms_d, h->tok, d.S,
                                    col, col_rows, out_d, h->probs, h->stream);
        }
        int rc = after_forward(h, e);
        if (rc) return rc;
    }
    if (h->rows_mode) {
        for (int b = 0; b < h->cur_B; b++)
            if (h->row_last[b] + 1 < d.S) h->row_next[b] = 1;
    } else if (col >= 0) {
        h->col_written[col] = 1;
    }
    return LLM_OK;
}

// Varlen prefill: validate lengths, build the packed-row map on the host.
int prep_varlen(llm_t *h, const int32_t *lens, int B, std::vector<int2> &rowmap, std::vector<int> &cu_last,
                int *Mout, int *Tmax)
{
    if (B < 1 || B > h->d.maxB) return fail(h, LLM_EINVAL, "B must be in [1, max_batch_size]");
    if (!lens) return fail(h, LLM_EINVAL, "lens is NULL");
    int64_t M = 0;
    int tmax = 0;
    for (int b = 0; b < B; b++) {
        if (lens[b] < 1 || lens[b] > h->d.S) return fail(h, LLM_EINVAL, "every length must be in [1, max_seq_len]");
        M += lens[b];
        tmax = std::max(tmax, (int)lens[b]);
    }
    rowmap.resize(M);
    cu_last.assign(2 * B + 1, 0);  // B + 1 starts, then B last rows
    int64_t m = 0;
    for (int b = 0; b < B; b++) {
        cu_last[b] = (int)m;
        for (int t = 0; t < lens[b]; t++, m++) rowmap[m] = make_int2(b, t);
        cu_last[B + 1 + b] = (int)m - 1;
    }
    cu_last[B] = (int)m;
    *Mout = (int)M;
    *Tmax = tmax;
    return LLM_OK;
}

// The forward of a varlen prefill whose packed tokens are in h->vtok.
int varlen_common(llm_t *h, const int32_t *lens, int B, const std::vector<int2> &rowmap,
                  const std::vector<int> &cu_last, int M, int Tmax)
{
    if (!h->dry) {
        int rc = ensure_ws(h, M);  // (callers run it before staging tokens as well)
        if (rc) return rc;
        if ((rc = kv_upload(h))) return rc;
        HIPC(h, hipMemcpyAsync(h->rowmap, rowmap.data(), (size_t)M * sizeof(int2), hipMemcpyHostToDevice, h->stream));
        HIPC(h, hipMemcpyAsync(h->cu, cu_last.data(), cu_last.size() * sizeof(int), hipMemcpyHostToDevice, h->stream));
        std::vector<int> last(B);
        for (int b = 0; b < B; b++) last[b] = lens[b] - 1;
        HIPC(h, hipMemcpyAsync(h->pos_rows, last.data(), (size_t)B * sizeof(int), hipMemcpyHostToDevice, h->stream));
        HIPC(h, launch_scatter_tokens(h->tok, h->d.S, M, h->rowmap, h->vtok, h->stream));
        Pass ps;
        ps.B = B;
        ps.M = M;
        ps.T = 1;
        ps.rowmap = h->rowmap;
        ps.cu = h->cu;
        ps.last_rows = h->cu + B + 1;
        ps.Tmax = Tmax;
        rc = after_forward(h, forward(h, ps));
        if (rc) return rc;
        HIPC(h, hipStreamSynchronize(h->stream));  // host copies of rowmap / lengths go out of scope
    }
    h->prefilled = true;
    h->logits_valid = true;
    h->rows_mode = true;
    h->cur_B = B;
    h->last_pos = -1;
    std::fill(h->col_written.begin(), h->col_written.end(), 0);
    for (int b = 0; b < h->d.maxB; b++) {
        h->row_last[b] = b < B ? lens[b] - 1 : -1;
        h->row_next[b] = 0;
    }
    return LLM_OK;
}

}  // namespace

// ===========================================================================
// C ABI
// ===========================================================================
// `reps` eager forward passes with HIP events around every kernel; ms_out
// receives the mean milliseconds per pass of each kernel class (ProfClass)
// and, last, the first-to-last event time.  prev_pos < 0: a prefill of B x T
// tokens at positions 0..T-1, else a decode step at prev_pos.
int profiled_forward(llm_t *h, int B, int T, int prev_pos, int reps, float *ms_out)
{
    int rc = kv_upload(h);
    if (rc) return rc;
    Prof pf;
    double acc[PC_N] = {0};
    hipError_t e = hipSuccess;
    for (int r = 0; r < reps && e == hipSuccess; r++) {
        pf.used = 0;
        const int *pos = nullptr;
        if (prev_pos >= 0) {
            e = launch_set_int(h->pos_dev, prev_pos, h->stream);
            h->dev_pos = prev_pos;
            pos = h->pos_dev;
        }
        if (e == hipSuccess) e = forward(h, uniform_pass(B, T, pos), &pf);
        if (e == hipSuccess) e = hipStreamSynchronize(h->stream);
        for (size_t i = 0; e == hipSuccess && i + 1 < pf.used; i += 2) {
            float ms = 0.f;
            e = hipEventElapsedTime(&ms, pf.ev[i], pf.ev[i + 1]);
            acc[pf.cls[i / 2]] += ms;
        }
        float all = 0.f;
        if (e == hipSuccess && pf.used >= 2) e = hipEventElapsedTime(&all, pf.ev[0], pf.ev[pf.used - 1]);
        acc[PC_N - 1] += all;
    }
    for (hipEvent_t ev : pf.ev) (void)hipEventDestroy(ev);
    if (e != hipSuccess) return fail(h, LLM_EDEVICE, std::string("profile: ") + hipGetErrorString(e));
    for (int c = 0; c < PC_N; c++) ms_out[c] = (float)(acc[c] / reps);
    return LLM_OK;
}

extern "C" {

int64_t llm_ffn_hidden(const llm_params *p)
{
    if (!check(p, nullptr).empty()) return -1;
    return ffn_width(p);
}

int64_t llm_kv_cache_bytes(const llm_params *p)
{
    Dims d;
    if (!check(p, &d).empty()) return -1;
    return (int64_t)d.NL * 2 * d.maxB * d.Hkv * d.S * d.hd * d.es;
}

int64_t llm_weight_bytes(const llm_params *p)
{
    Dims d;
    if (!check(p, &d).empty()) return -1;
    int64_t per_layer = d.Nqkv * d.D + (int64_t)d.D * d.H * d.hd + 3 * (int64_t)d.F * d.D;
    return d.es * (d.NL * per_layer + (int64_t)d.V * d.D);
}

int llm_check_params(const llm_params *p) { return check(p, nullptr).empty() ? LLM_OK : LLM_EINVAL; }

static llm_t *new_handle(const llm_params *p, const Dims &d)
{
    llm_t *h = new (std::nothrow) llm_t();
    if (!h) return nullptr;
    h->p = *p;
    h->d = d;
    h->col_written.assign(d.S, 0);
    h->row_last.assign(d.maxB, -1);
    h->row_next.assign(d.maxB, 0);
    const char *ng = std::getenv("LLM_NO_GRAPH");
    h->use_graph = !(ng && ng[0] == '1');
    return h;
}

// Set up the paged-cache fields of a new handle (sizes only).
static void set_paging(llm_t *h, const llm_paging *pg)
{
    h->bs = pg->block_size;
    h->bshift = 0;
    while ((1 << h->bshift) < h->bs) h->bshift++;
    h->bt_ld = (h->d.S + h->bs - 1) / h->bs;
    h->kv_blocks = pg->num_blocks;
    h->kv_util = pg->gpu_memory_utilization;
}

static int create_dry(const llm_params *p, const llm_paging *pg, llm_t **out)
{
    if (!out) return LLM_EINVAL;
    *out = nullptr;
    Dims d;
    if (!check(p, &d).empty()) return LLM_EINVAL;
    if (pg && !check_paging(d, pg, true).empty()) return LLM_EINVAL;
    llm_t *h = new_handle(p, d);
    if (!h) return LLM_ENOMEM;
    h->dry = true;
    if (pg) {
        set_paging(h, pg);
        init_pages(h, pg->num_blocks);
    }
    *out = h;
    return LLM_OK;
}

static int create(const llm_params *p, const llm_paging *pg, uint64_t seed, void *hip_stream, llm_t **out)
{
    if (!out) return LLM_EINVAL;
    *out = nullptr;
    Dims d;
    std::string why = check(p, &d);
    if (why.empty() && pg) why = check_paging(d, pg, false);
    if (!why.empty()) {
        fprintf(stderr, "llm_create: %s\n", why.c_str());
        return LLM_EINVAL;
    }
    llm_t *h = new_handle(p, d);
    if (!h) return LLM_ENOMEM;
    if (pg) set_paging(h, pg);
    if (hip_stream) {
        h->stream = (hipStream_t)hip_stream;
    } else {
        if (hipStreamCreateWithFlags(&h->stream, hipStreamNonBlocking) != hipSuccess) {
            delete h;
            return LLM_EDEVICE;
        }
        h->own_stream = true;
    }
    int rc = create_impl(h, seed);
    if (rc != LLM_OK) {
        fprintf(stderr, "llm_create: %s\n", h->err.c_str());
        (void)hipDeviceSynchronize();
        release(h);
        delete h;
        return rc;
    }
    *out = h;
    return LLM_OK;
}

int llm_create_dry(const llm_params *p, llm_t **out) { return create_dry(p, nullptr, out); }

int llm_create(const llm_params *p, uint64_t seed, void *hip_stream, llm_t **out)
{
    return create(p, nullptr, seed, hip_stream, out);
}

int64_t llm_kv_block_bytes(const llm_params *p, int32_t block_size)
{
    Dims d;
    if (!check(p, &d).empty() || block_size < 1) return -1;
    return block_bytes(d, block_size);
}

int llm_create_paged(const llm_params *p, const llm_paging *pg, uint64_t seed, void *hip_stream, llm_t **out)
{
    if (!pg) {
        if (out) *out = nullptr;
        return LLM_EINVAL;
    }
    return create(p, pg, seed, hip_stream, out);
}

int llm_create_paged_dry(const llm_params *p, const llm_paging *pg, llm_t **out)
{
    if (!pg) {
        if (out) *out = nullptr;
        return LLM_EINVAL;
    }
    return create_dry(p, pg, out);
}

int32_t llm_kv_num_blocks(const llm_t *h) { return h && h->bs ? h->kv_blocks : 0; }

int32_t llm_kv_free_blocks(const llm_t *h) { return h && h->bs ? (int32_t)h->free_ids.size() : 0; }

int32_t llm_kv_table_width(const llm_t *h) { return h && h->bs ? h->bt_ld : 0; }

int llm_kv_block_table(llm_t *h, int32_t row, int32_t *out, int32_t n)
{
    int rc = guard(h);
    if (rc) return rc;
    if (!h->bs) return fail(h, LLM_EINVAL, "not a paged handle");
    if (row < 0 || row >= h->d.maxB) return fail(h, LLM_EINVAL, "row must be in [0, max_batch_size)");
    if (!out || n < 0 || n > h->bt_ld) return fail(h, LLM_EINVAL, "n must be in [0, table width]");
    memcpy(out, h->btab.data() + (size_t)row * h->bt_ld, (size_t)n * sizeof(int32_t));
    return LLM_OK;
}

int llm_kv_set_block_table(llm_t *h, int32_t row, const int32_t *blocks, int32_t n)
{
    int rc = guard(h);
    if (rc) return rc;
    if (!h->bs) return fail(h, LLM_EINVAL, "not a paged handle");
    if (row < 0 || row >= h->d.maxB) return fail(h, LLM_EINVAL, "row must be in [0, max_batch_size)");
    if (n < 0 || n > h->bt_ld || (n > 0 && !blocks)) return fail(h, LLM_EINVAL, "n must be in [0, table width]");
    std::set<int> seen;
    for (int i = 0; i < n; i++) {
        const int id = blocks[i];
        if (id < 0 || id >= h->kv_blocks) return fail(h, LLM_EINVAL, "block id out of [0, num_blocks)");
        if (!seen.insert(id).second) return fail(h, LLM_EINVAL, "a block id appears twice");
        if (h->owner[id] >= 0 && h->owner[id] != row) return fail(h, LLM_EINVAL, "a block is held by another row");
    }
    int *t = h->btab.data() + (size_t)row * h->bt_ld;
    for (int i = 0; i < h->bt_ld; i++)
        if (t[i] >= 0) {
            h->owner[t[i]] = -1;
            h->free_ids.insert(t[i]);
            t[i] = -1;
        }
    for (int i = 0; i < n; i++) {
        t[i] = blocks[i];
        h->owner[t[i]] = row;
        h->free_ids.erase(t[i]);
    }
    h->btab_dirty = true;
    return LLM_OK;
}

void llm_destroy(llm_t *h)
{
    if (!h) return;
    if (!h->dry) {
        if (h->stream) (void)hipStreamSynchronize(h->stream);
        release(h);
    }
    delete h;
}

const char *llm_last_error(const llm_t *h) { return h ? h->err.c_str() : static_call_error(); }

void *llm_get_stream(llm_t *h) { return h ? (void *)h->stream : nullptr; }

int llm_prefill(llm_t *h, const int32_t *tokens, int32_t B, int32_t T)
{
    int rc = guard(h);
    if (rc) return rc;
    if ((rc = check_prefill_args(h, B, T))) return rc;
    if (!tokens) return fail(h, LLM_EINVAL, "tokens is NULL");
    if (!tokens_ok(tokens, (int64_t)B * T, h->d.V)) return fail(h, LLM_EINVAL, "token id out of [0, vocab)");
    if ((rc = kv_reserve_uniform(h, B, 0, T, true))) return rc;
    if (!h->dry) {
        HIPC(h, hipMemcpy2DAsync(h->tok, (size_t)h->d.S * 4, tokens, (size_t)T * 4, (size_t)T * 4, B,
                                 hipMemcpyHostToDevice, h->stream));
        HIPC(h, hipStreamSynchronize(h->stream));
    }
    return prefill_common(h, B, T);
}

int llm_prefill_d(llm_t *h, const int32_t *tokens_d, int32_t B, int32_t T)
{
    int rc = guard(h);
    if (rc) return rc;
    if ((rc = check_prefill_args(h, B, T))) return rc;
    if (!tokens_d) return fail(h, LLM_EINVAL, "tokens is NULL");
    if (h->dry) return fail(h, LLM_ESTATE, "dry handle has no device memory");
    if ((rc = kv_reserve_uniform(h, B, 0, T, true))) return rc;
    HIPC(h, hipMemcpy2DAsync(h->tok, (size_t)h->d.S * 4, tokens_d, (size_t)T * 4, (size_t)T * 4, B,
                             hipMemcpyDeviceToDevice, h->stream));
    return prefill_common(h, B, T);
}

int llm_prefill_at(llm_t *h, int32_t start_pos, const int32_t *tokens, int32_t B, int32_t T)
{
    int rc = guard(h);
    if (rc) return rc;
    if ((rc = check_prefill_args(h, B, T, start_pos))) return rc;
    if (!tokens) return fail(h, LLM_EINVAL, "tokens is NULL");
    if (!tokens_ok(tokens, (int64_t)B * T, h->d.V)) return fail(h, LLM_EINVAL, "token id out of [0, vocab)");
    if ((rc = kv_reserve_uniform(h, B, start_pos, start_pos + T, start_pos == 0))) return rc;
    if (!h->dry) {
        HIPC(h, hipMemcpy2DAsync(h->tok + start_pos, (size_t)h->d.S * 4, tokens, (size_t)T * 4, (size_t)T * 4, B,
                                 hipMemcpyHostToDevice, h->stream));
        HIPC(h, hipStreamSynchronize(h->stream));
    }
    return prefill_common(h, B, T, start_pos);
}

int llm_prefill_at_d(llm_t *h, int32_t start_pos, const int32_t *tokens_d, int32_t B, int32_t T)
{
    int rc = guard(h);
    if (rc) return rc;
    if ((rc = check_prefill_args(h, B, T, start_pos))) return rc;
    if (!tokens_d) return fail(h, LLM_EINVAL, "tokens is NULL");
    if (h->dry) return fail(h, LLM_ESTATE, "dry handle has no device memory");
    if ((rc = kv_reserve_uniform(h, B, start_pos, start_pos + T, start_pos == 0))) return rc;
    HIPC(h, hipMemcpy2DAsync(h->tok + start_pos, (size_t)h->d.S * 4, tokens_d, (size_t)T * 4, (size_t)T * 4, B,
                             hipMemcpyDeviceToDevice, h->stream));
    return prefill_common(h, B, T, start_pos);
}

int llm_prefill_varlen(llm_t *h, const int32_t *tokens, const int32_t *lens, int32_t B)
{
    int rc = guard(h);
    if (rc) return rc;
    std::vector<int2> rowmap;
    std::vector<int> cu_last;
    int M = 0, Tmax = 0;
    if ((rc = prep_varlen(h, lens, B, rowmap, cu_last, &M, &Tmax))) return rc;
    if (!tokens) return fail(h, LLM_EINVAL, "tokens is NULL");
    if (!tokens_ok(tokens, M, h->d.V)) return fail(h, LLM_EINVAL, "token id out of [0, vocab)");
    if ((rc = kv_reserve(h, B, std::vector<int>(B, 0), std::vector<int>(lens, lens + B), true))) return rc;
    if (!h->dry) {
        if ((rc = ensure_ws(h, M))) return rc;
        HIPC(h, hipMemcpyAsync(h->vtok, tokens, (size_t)M * 4, hipMemcpyHostToDevice, h->stream));
    }
    return varlen_common(h, lens, B, rowmap, cu_last, M, Tmax);
}

int llm_prefill_varlen_d(llm_t *h, const int32_t *tokens_d, const int32_t *lens, int32_t B)
{
    int rc = guard(h);
    if (rc) return rc;
    std::vector<int2> rowmap;
    std::vector<int> cu_last;
    int M = 0, Tmax = 0;
    if ((rc = prep_varlen(h, lens, B, rowmap, cu_last, &M, &Tmax))) return rc;
    if (!tokens_d) return fail(h, LLM_EINVAL, "tokens is NULL");
    if (h->dry) return fail(h, LLM_ESTATE, "dry handle has no device memory");
    if ((rc = kv_reserve(h, B, std::vector<int>(B, 0), std::vector<int>(lens, lens + B), true))) return rc;
    if ((rc = ensure_ws(h, M))) return rc;
    HIPC(h, hipMemcpyAsync(h->vtok, tokens_d, (size_t)M * 4, hipMemcpyDeviceToDevice, h->stream));
    return varlen_common(h, lens, B, rowmap, cu_last, M, Tmax);
}

int llm_decode_rows(llm_t *h)
{
    int rc = guard(h);
    if (rc) return rc;
    if (!h->prefilled || !h->rows_mode) return fail(h, LLM_ESTATE, "per-row decode needs a varlen prefill first");
    const int B = h->cur_B;
    for (int b = 0; b < B; b++) {
        if (h->row_last[b] + 1 >= h->d.S) return fail(h, LLM_EINVAL, "a row has reached max_seq_len");
        if (!h->row_next[b]) return fail(h, LLM_ESTATE, "a row's next token column has not been written");
    }
    {
        std::vector<int> rd(B), en(B);
        for (int b = 0; b < B; b++) {
            rd[b] = h->row_last[b] + 1;
            en[b] = h->row_last[b] + 2;
        }
        if ((rc = kv_reserve(h, B, rd, en, false))) return rc;
    }
    if (!h->dry) {
        if ((rc = kv_upload(h))) return rc;
        // each row moves to its next position, then the step runs at pos_rows[b]
        HIPC(h, launch_inc_ints(h->pos_rows, B, h->stream));
        Pass ps;
        ps.B = B;
        ps.M = B;
        ps.T = 1;
        ps.pos_rows = h->pos_rows;
        if (h->use_graph) {
            if (!h->gexec_rows || h->graph_rows_B != B) {
                if (h->gexec_rows) {
                    (void)hipGraphExecDestroy(h->gexec_rows);
                    h->gexec_rows = nullptr;
                }
                hipGraph_t graph = nullptr;
                HIPC(h, hipStreamBeginCapture(h->stream, hipStreamCaptureModeRelaxed));
                hipError_t fe = forward(h, ps);
                hipError_t ce = hipStreamEndCapture(h->stream, &graph);
                if (fe != hipSuccess) return fail(h, LLM_EDEVICE, std::string("capture: ") + hipGetErrorString(fe));
                if (ce != hipSuccess) return fail(h, LLM_EDEVICE, std::string("end capture: ") + hipGetErrorString(ce));
                hipError_t ie = hipGraphInstantiate(&h->gexec_rows, graph, nullptr, nullptr, 0);
                (void)hipGraphDestroy(graph);
                if (ie != hipSuccess) return fail(h, LLM_EDEVICE, std::string("instantiate: ") + hipGetErrorString(ie));
                h->graph_rows_B = B;
            }
            HIPC(h, hipGraphLaunch(h->gexec_rows, h->stream));
        } else {
            rc = after_forward(h, forward(h, ps));
            if (rc) return rc;
        }
    }
    for (int b = 0; b < B; b++) {
        h->row_last[b]++;
        h->row_next[b] = 0;
    }
    h->logits_valid = true;
    return LLM_OK;
}

int llm_set_tokens_rows(llm_t *h, const int32_t *tokens, const uint8_t *mask)
{
    int rc = guard(h);
    if (rc) return rc;
    if (!h->prefilled || !h->rows_mode) return fail(h, LLM_ESTATE, "per-row tokens need a varlen prefill first");
    if (!tokens) return fail(h, LLM_EINVAL, "tokens is NULL");
    const int B = h->cur_B;
    for (int b = 0; b < B; b++) {
        const bool use = !mask || mask[b];
        if (use && (tokens[b] < 0 || tokens[b] >= h->d.V)) return fail(h, LLM_EINVAL, "token id out of [0, vocab)");
        if (use && h->row_last[b] + 1 >= h->d.S) return fail(h, LLM_EINVAL, "a row has no column left");
    }
    if (!h->dry) {
        HIPC(h, hipMemcpyAsync(h->stage_i32, tokens, (size_t)B * 4, hipMemcpyHostToDevice, h->stream));
        if (mask) HIPC(h, hipMemcpyAsync(h->stage_mask, mask, (size_t)B, hipMemcpyHostToDevice, h->stream));
        HIPC(h, launch_set_tokens_rows(h->tok, h->d.S, B, h->pos_rows, h->stage_i32, mask ? h->stage_mask : nullptr,
                                       h->stream));
        HIPC(h, hipStreamSynchronize(h->stream));
    }
    for (int b = 0; b < B; b++)
        if (!mask || mask[b]) h->row_next[b] = 1;
    return LLM_OK;
}

int llm_decode(llm_t *h, int32_t prev_pos)
{
    int rc = guard(h);
    if (rc) return rc;
    if (!h->prefilled) return fail(h, LLM_ESTATE, "decode before prefill");
    if (h->rows_mode) return fail(h, LLM_ESTATE, "rows are at different positions: use llm_decode_rows");
    if (prev_pos < 1 || prev_pos >= h->d.S) return fail(h, LLM_EINVAL, "prev_pos must be in [1, max_seq_len)");
    if (prev_pos > h->last_pos + 1) return fail(h, LLM_ESTATE, "prev_pos skips positions whose KV is not written");
    if (!h->col_written[prev_pos]) return fail(h, LLM_ESTATE, "token column prev_pos has not been written");
    if ((rc = kv_reserve_uniform(h, h->cur_B, prev_pos, prev_pos + 1, false))) return rc;
    if (!h->dry) {
        if ((rc = kv_upload(h))) return rc;
        // each step moves the device position on by one, so consecutive
        // steps need no position write
        if (h->dev_pos != prev_pos) {
            h->dev_pos = -1;
            HIPC(h, launch_set_int(h->pos_dev, prev_pos, h->stream));
        }
        const int B = h->cur_B;
        Pass ps = uniform_pass(B, 1, h->pos_dev);
        ps.advance = true;
        if (h->use_graph) {
            if (!h->gexec || h->graph_B != B) {
                if (h->gexec) {
                    (void)hipGraphExecDestroy(h->gexec);
                    h->gexec = nullptr;
                }
                hipGraph_t graph = nullptr;
                HIPC(h, hipStreamBeginCapture(h->stream, hipStreamCaptureModeRelaxed));
                hipError_t fe = forward(h, ps);
                hipError_t ce = hipStreamEndCapture(h->stream, &graph);
                if (fe != hipSuccess) return fail(h, LLM_EDEVICE, std::string("capture: ") + hipGetErrorString(fe));
                if (ce != hipSuccess) return fail(h, LLM_EDEVICE, std::string("end capture: ") + hipGetErrorString(ce));
                hipError_t ie = hipGraphInstantiate(&h->gexec, graph, nullptr, nullptr, 0);
                (void)hipGraphDestroy(graph);
                if (ie != hipSuccess) return fail(h, LLM_EDEVICE, std::string("instantiate: ") + hipGetErrorString(ie));
                h->graph_B = B;
            }
            HIPC(h, hipGraphLaunch(h->gexec, h->stream));
        } else {
            rc = after_forward(h, forward(h, ps));
            if (rc) return rc;
        }
        h->dev_pos = prev_pos + 1;
    }
    h->last_pos = prev_pos;
    h->logits_valid = true;
    return LLM_OK;
}

int llm_sample(llm_t *h, float temperature, float top_p, const float *uniforms, int32_t *out_tokens)
{
    int rc = guard(h);
    if (rc) return rc;
    if (h->dry && out_tokens) return fail(h, LLM_ESTATE, "dry handle returns no tokens");
    bool have_u = uniforms != nullptr;
    if ((rc = sample_check(h, temperature, top_p, have_u))) return rc;
    if (!h->dry && have_u && temperature > 0.f) {
        // host uniforms go through pinned staging, so the call need not wait
        // for the copy; the previous call's copy must have read the staging
        HIPC(h, hipEventSynchronize(h->uni_ev));
        memcpy(h->uni_stage, uniforms, (size_t)h->cur_B * sizeof(float));
        HIPC(h, hipMemcpyAsync(h->uni, h->uni_stage, (size_t)h->cur_B * sizeof(float), hipMemcpyHostToDevice,
                               h->stream));
        HIPC(h, hipEventRecord(h->uni_ev, h->stream));
    }
    rc = sample_common(h, temperature, top_p, h->uni, have_u, out_tokens ? h->outtok : nullptr);
    if (rc) return rc;
    if (out_tokens) {
        HIPC(h, hipMemcpyAsync(out_tokens, h->outtok, (size_t)h->cur_B * sizeof(int32_t),
                               hipMemcpyDeviceToHost, h->stream));
        HIPC(h, hipStreamSynchronize(h->stream));
    }
    return LLM_OK;
}

int llm_sample_d(llm_t *h, float temperature, float top_p, const float *uniforms_d, int32_t *out_tokens_d)
{
    int rc = guard(h);
    if (rc) return rc;
    if (h->dry && (uniforms_d || out_tokens_d)) return fail(h, LLM_ESTATE, "dry handle has no device memory");
    return sample_common(h, temperature, top_p, uniforms_d, uniforms_d != nullptr, out_tokens_d);
}

int llm_set_tokens(llm_t *h, int32_t pos, const int32_t *tokens, const uint8_t *mask)
{
    int rc = guard(h);
    if (rc) return rc;
    if (!h->prefilled) return fail(h, LLM_ESTATE, "set_tokens before prefill");
    if (h->rows_mode) return fail(h, LLM_ESTATE, "rows are at different positions: use llm_set_tokens_rows");
    if (pos < 0 || pos >= h->d.S) return fail(h, LLM_EINVAL, "pos must be in [0, max_seq_len)");
    if (!tokens) return fail(h, LLM_EINVAL, "tokens is NULL");
    const int B = h->cur_B;
    bool all = true;
    for (int b = 0; b < B; b++) {
        bool use = !mask || mask[b];
        all = all && use;
        if (use && (tokens[b] < 0 || tokens[b] >= h->d.V)) return fail(h, LLM_EINVAL, "token id out of [0, vocab)");
    }
    if (!h->dry) {
        HIPC(h, hipMemcpyAsync(h->stage_i32, tokens, (size_t)B * 4, hipMemcpyHostToDevice, h->stream));
        if (mask) HIPC(h, hipMemcpyAsync(h->stage_mask, mask, (size_t)B, hipMemcpyHostToDevice, h->stream));
        HIPC(h, launch_set_tokens(h->tok, h->d.S, B, pos, h->stage_i32, mask ? h->stage_mask : nullptr, h->stream));
        HIPC(h, hipStreamSynchronize(h->stream));
    }
    if (all) h->col_written[pos] = 1;
    return LLM_OK;
}

int llm_set_tokens_d(llm_t *h, int32_t pos, const int32_t *tokens_d, const uint8_t *mask_d)
{
    int rc = guard(h);
    if (rc) return rc;
    if (!h->prefilled) return fail(h, LLM_ESTATE, "set_tokens before prefill");
    if (h->rows_mode) return fail(h, LLM_ESTATE, "rows are at different positions: use llm_set_tokens_rows");
    if (pos < 0 || pos >= h->d.S) return fail(h, LLM_EINVAL, "pos must be in [0, max_seq_len)");
    if (!tokens_d) return fail(h, LLM_EINVAL, "tokens is NULL");
    if (h->dry) return fail(h, LLM_ESTATE, "dry handle has no device memory");
    HIPC(h, launch_set_tokens(h->tok, h->d.S, h->cur_B, pos, tokens_d, mask_d, h->stream));
    if (!mask_d) h->col_written[pos] = 1;
    return LLM_OK;
}

int llm_profile_decode(llm_t *h, int32_t prev_pos, int32_t reps, float *ms_out)
{
    int rc = guard(h);
    if (rc) return rc;
    if (!ms_out || reps < 1) return fail(h, LLM_EINVAL, "bad arguments");
    if (h->dry) return fail(h, LLM_ESTATE, "dry handle has no device memory");
    if (!h->prefilled) return fail(h, LLM_ESTATE, "decode before prefill");
    if (h->rows_mode) return fail(h, LLM_ESTATE, "rows are at different positions");
    if (prev_pos < 1 || prev_pos >= h->d.S) return fail(h, LLM_EINVAL, "prev_pos must be in [1, max_seq_len)");
    if (prev_pos > h->last_pos + 1) return fail(h, LLM_ESTATE, "prev_pos skips positions whose KV is not written");
    if (!h->col_written[prev_pos]) return fail(h, LLM_ESTATE, "token column prev_pos has not been written");
    if ((rc = kv_reserve_uniform(h, h->cur_B, prev_pos, prev_pos + 1, false))) return rc;
    rc = profiled_forward(h, h->cur_B, 1, prev_pos, reps, ms_out);
    if (rc) return rc;
    h->last_pos = prev_pos;
    h->logits_valid = true;
    return LLM_OK;
}

int llm_profile_prefill(llm_t *h, const int32_t *tokens_d, int32_t B, int32_t T, int32_t reps, float *ms_out)
{
    int rc = guard(h);
    if (rc) return rc;
    if ((rc = check_prefill_args(h, B, T))) return rc;
    if (!tokens_d || !ms_out || reps < 1) return fail(h, LLM_EINVAL, "bad arguments");
    if (h->dry) return fail(h, LLM_ESTATE, "dry handle has no device memory");
    if ((rc = kv_reserve_uniform(h, B, 0, T, true))) return rc;
    HIPC(h, hipMemcpy2DAsync(h->tok, (size_t)h->d.S * 4, tokens_d, (size_t)T * 4, (size_t)T * 4, B,
                             hipMemcpyDeviceToDevice, h->stream));
    if ((rc = ensure_ws(h, (int64_t)B * T))) return rc;
    if ((rc = profiled_forward(h, B, T, -1, reps, ms_out))) return rc;
    h->prefilled = true;
    h->logits_valid = true;
    h->cur_B = B;
    h->last_pos = T - 1;
    std::fill(h->col_written.begin(), h->col_written.end(), 0);
    std::fill(h->col_written.begin(), h->col_written.begin() + T, 1);
    return LLM_OK;
}

// Launches of one timing pass of llm_profile_projections: kind 0..4 is that
// product over every layer (the head once) `reps` times; kind 5 the whole
// decode sequence of products in forward order `reps` times.
hipError_t projection_pass(llm_t *h, int kind, int reps, bool fused, int *launches)
{
    const int kinds[5] = {MAT_QKV, MAT_O, MAT_W13, MAT_W2, MAT_HEAD};
    const int B = h->cur_B, NL = h->d.NL;
    hipError_t e = hipSuccess;
    *launches = 0;
    // the products take the forms of a decode step: wo, and w2 but the last
    // layer's, may hand split-K partials to the next normalisation launch
    // (not run here: only the products are timed)
    int unused = 0;
    auto hand = [&](int mat, int l) -> int * {
        return !fused && (mat == MAT_O || (mat == MAT_W2 && l + 1 < NL)) ? &unused : nullptr;
    };
    for (int r = 0; r < reps && e == hipSuccess; r++) {
        if (kind < 5) {
            const int per_rep = kinds[kind] == MAT_HEAD ? 1 : NL;
            for (int l = 0; l < per_rep && e == hipSuccess; l++, ++*launches)
                e = product(h, l, kinds[kind], uniform_pass(B, 1, h->pos_dev), fused, hand(kinds[kind], l));
        } else {
            for (int l = 0; l < NL && e == hipSuccess; l++)
                for (int k = 0; k < 4 && e == hipSuccess; k++, ++*launches)
                    e = product(h, l, kinds[k], uniform_pass(B, 1, h->pos_dev), fused, hand(kinds[k], l));
            if (e == hipSuccess) e = product(h, 0, MAT_HEAD, uniform_pass(B, 1, h->pos_dev), fused);
            ++*launches;
        }
    }
    return e;
}

int llm_profile_projections(llm_t *h, int32_t reps, float *us_out)
{
    int rc = guard(h);
    if (rc) return rc;
    if (!us_out || reps < 1) return fail(h, LLM_EINVAL, "bad arguments");
    if (h->dry) return fail(h, LLM_ESTATE, "dry handle has no device memory");
    if (h->d.dtype != LLM_F16) return fail(h, LLM_EINVAL, "projection timing is for fp16 models");
    if (!h->prefilled) return fail(h, LLM_ESTATE, "projection timing before prefill");
    if (h->rows_mode) return fail(h, LLM_ESTATE, "rows are at different positions");
    if ((rc = kv_reserve_uniform(h, h->cur_B, h->last_pos + 1, h->last_pos + 1, false))) return rc;
    if ((rc = kv_upload(h))) return rc;
    const bool fused = fuse_norm(h, h->cur_B);
    hipEvent_t ev[2] = {nullptr, nullptr};
    hipError_t e = hipEventCreate(&ev[0]);
    if (e == hipSuccess) e = hipEventCreate(&ev[1]);
    if (e == hipSuccess) e = launch_set_int(h->pos_dev, h->last_pos, h->stream);
    h->dev_pos = h->last_pos;
    // each pass is captured once and replayed, as a decode step is, so the
    // host's launch rate does not pace the short products
    for (int k = 0; k < 6 && e == hipSuccess; k++) {
        hipGraph_t graph = nullptr;
        hipGraphExec_t exec = nullptr;
        int launches = 0;
        e = hipStreamBeginCapture(h->stream, hipStreamCaptureModeRelaxed);
        if (e == hipSuccess) {
            hipError_t pe = projection_pass(h, k, reps, fused, &launches);
            e = hipStreamEndCapture(h->stream, &graph);
            if (pe != hipSuccess) e = pe;
        }
        if (e == hipSuccess) e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
        if (e == hipSuccess) e = hipGraphLaunch(exec, h->stream);  // warm-up
        if (e == hipSuccess) e = hipEventRecord(ev[0], h->stream);
        if (e == hipSuccess) e = hipGraphLaunch(exec, h->stream);
        if (e == hipSuccess) e = hipEventRecord(ev[1], h->stream);
        if (e == hipSuccess) e = hipEventSynchronize(ev[1]);
        float ms = 0.f;
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, ev[0], ev[1]);
        us_out[k] = launches ? ms * 1e3f / (float)launches : 0.f;
        if (exec) (void)hipGraphExecDestroy(exec);
        if (graph) (void)hipGraphDestroy(graph);
    }
    for (hipEvent_t x : ev)
        if (x) (void)hipEventDestroy(x);
    // the workspace, logits and the cache entry at last_pos now hold junk
    h->prefilled = false;
    h->logits_valid = false;
    if (e != hipSuccess) return fail(h, LLM_EDEVICE, std::string("profile: ") + hipGetErrorString(e));
    return LLM_OK;
}

int llm_get_logits(llm_t *h, float *out)
{
    int rc = guard(h);
    if (rc) return rc;
    if (!out) return fail(h, LLM_EINVAL, "out is NULL");
    if (h->dry) return fail(h, LLM_ESTATE, "dry handle has no logits");
    if (!h->logits_valid) return fail(h, LLM_ESTATE, "no logits yet");
    HIPC(h, hipMemcpyAsync(out, h->logits, (size_t)h->cur_B * h->d.V * sizeof(float), hipMemcpyDeviceToHost,
                           h->stream));
    HIPC(h, hipStreamSynchronize(h->stream));
    return LLM_OK;
}

int llm_get_logits_d(llm_t *h, float *out_d)
{
    int rc = guard(h);
    if (rc) return rc;
    if (!out_d) return fail(h, LLM_EINVAL, "out is NULL");
    if (h->dry) return fail(h, LLM_ESTATE, "dry handle has no logits");
    if (!h->logits_valid) return fail(h, LLM_ESTATE, "no logits yet");
    HIPC(h, hipMemcpyAsync(out_d, h->logits, (size_t)h->cur_B * h->d.V * sizeof(float),
                           hipMemcpyDeviceToDevice, h->stream));
    return LLM_OK;
}

int llm_get_tokens(llm_t *h, int32_t n_cols, int32_t *out)
{
    int rc = guard(h);
    if (rc) return rc;
    if (!out || n_cols < 1 || n_cols > h->d.S) return fail(h, LLM_EINVAL, "n_cols must be in [1, max_seq_len]");
    if (h->dry || !h->prefilled) return fail(h, LLM_ESTATE, "no token buffer yet");
    HIPC(h, hipMemcpy2DAsync(out, (size_t)n_cols * 4, h->tok, (size_t)h->d.S * 4, (size_t)n_cols * 4, h->cur_B,
                             hipMemcpyDeviceToHost, h->stream));
    HIPC(h, hipStreamSynchronize(h->stream));
    return LLM_OK;
}

int llm_sample_probs(llm_t *h, const float *probs, int32_t B, float top_p, const float *uniforms, int32_t *out)
{
    int rc = guard(h);
    if (rc) return rc;
    if (B < 1 || B > h->d.maxB) return fail(h, LLM_EINVAL, "B must be in [1, max_batch_size]");
    if (!probs || !uniforms || !out) return fail(h, LLM_EINVAL, "NULL argument");
    if (!(top_p > 0.f && top_p <= 1.f)) return fail(h, LLM_EINVAL, "top_p must be in (0, 1]");
    if (h->dry) return fail(h, LLM_ESTATE, "dry handle has no device memory");
    HIPC(h, hipMemcpyAsync(h->probs, probs, (size_t)B * h->d.V * sizeof(float), hipMemcpyHostToDevice, h->stream));
    HIPC(h, hipMemcpyAsync(h->uni, uniforms, (size_t)B * sizeof(float), hipMemcpyHostToDevice, h->stream));
    HIPC(h, launch_sample_top_p(h->probs, false, 1.f, B, h->d.V, top_p, h->uni, h->tok, h->d.S, -1, nullptr,
                                h->outtok, nullptr, h->stream));
    HIPC(h, hipMemcpyAsync(out, h->outtok, (size_t)B * sizeof(int32_t), hipMemcpyDeviceToHost, h->stream));
    HIPC(h, hipStreamSynchronize(h->stream));
    h->logits_valid = false;  // the probability buffer no longer matches the logits
    return LLM_OK;
}

int llm_sync(llm_t *h)
{
    int rc = guard(h);
    if (rc) return rc;
    if (!h->dry) HIPC(h, hipStreamSynchronize(h->stream));
    return LLM_OK;
}

int llm_read_weights(llm_t *h, int32_t tensor_id, int64_t first, int64_t count, void *out)
{
    int rc = guard(h);
    if (rc) return rc;
    if (h->dry) return fail(h, LLM_ESTATE, "dry handle has no weights");
    const Dims &d = h->d;
    int mat, layer = 0, which = 0;
    int64_t rows, cols;
    if (tensor_id == 0) { mat = MAT_EMB; rows = d.V; cols = d.D; }
    else if (tensor_id == 1) { mat = MAT_HEAD; rows = d.V; cols = d.D; }
    else if (tensor_id >= 16 && (tensor_id - 16) / 8 < d.NL && (tensor_id - 16) % 8 < 7) {
        layer = (tensor_id - 16) / 8;
        which = (tensor_id - 16) % 8;
        const int wm[7] = {MAT_QKV, MAT_QKV, MAT_QKV, MAT_O, MAT_W13, MAT_W2, MAT_W13};
        mat = wm[which];
        int64_t r7[7] = {(int64_t)d.H * d.hd, (int64_t)d.Hkv * d.hd, (int64_t)d.Hkv * d.hd, d.D, d.F, d.D, d.F};
        rows = r7[which];
        cols = mat_cols(d, mat);
    } else {
        return fail(h, LLM_EINVAL, "unknown tensor id");
    }
    if (!out || first < 0 || count < 1 || first + count > rows * cols) return fail(h, LLM_EINVAL, "bad range");
    void *tmp = nullptr;
    HIPM(h, hipMalloc(&tmp, count * d.es));
    hipError_t e = launch_read_weights(mat_ptr(h, layer, mat), d.dtype, mat, mat_rows(d, mat), cols, which,
                                       d.H, d.Hkv, d.hd, d.F, first, count, tmp, h->stream);
    if (e == hipSuccess) e = hipMemcpyAsync(out, tmp, count * d.es, hipMemcpyDeviceToHost, h->stream);
    if (e == hipSuccess) e = hipStreamSynchronize(h->stream);
    (void)hipFree(tmp);
    if (e != hipSuccess) return fail(h, LLM_EDEVICE, std::string("read_weights: ") + hipGetErrorString(e));
    return LLM_OK;
}

static int op_begin(llm_t *h)
{
    int rc = guard(h);
    if (rc) return rc;
    if (h->dry) return fail(h, LLM_ESTATE, "dry handle has no device memory");
    HIPC(h, hipDeviceSynchronize());
    return LLM_OK;
}

static int op_end(llm_t *h, hipError_t e)
{
    if (e != hipSuccess) return fail(h, LLM_EDEVICE, std::string("op launch: ") + hipGetErrorString(e));
    HIPC(h, hipStreamSynchronize(h->stream));
    return LLM_OK;
}

int llm_op_rmsnorm(llm_t *h, const void *x_d, int32_t M, void *y_d)
{
    int rc = op_begin(h);
    if (rc) return rc;
    if (!x_d || !y_d || M < 1) return fail(h, LLM_EINVAL, "bad arguments");
    return op_end(h, launch_rmsnorm(x_d, h->d.D, h->norm_w, M, h->d.D, h->p.norm_eps, h->d.dtype, y_d, h->stream));
}

int llm_op_linear(llm_t *h, int32_t layer, int32_t mat, const void *x_d, int32_t M, void *y_d)
{
    int rc = op_begin(h);
    if (rc) return rc;
    if (!x_d || !y_d || M < 1) return fail(h, LLM_EINVAL, "bad arguments");
    if (mat < 0 || mat > MAT_HEAD || (mat != MAT_HEAD && (layer < 0 || layer >= h->d.NL)))
        return fail(h, LLM_EINVAL, "bad matrix or layer");
    if (mat == MAT_HEAD) layer = 0;
    Epilogue ep = make_ep(EP_STORE, y_d, mat_rows(h->d, mat));
    return op_end(h, run_linear(h, layer, mat, x_d, mat_cols(h->d, mat), M, ep));
}

int llm_op_kv_write(llm_t *h, int32_t layer, const void *k_d, const void *v_d, int32_t B, int32_t T, int32_t pos0)
{
    int rc = op_begin(h);
    if (rc) return rc;
    const Dims &d = h->d;
    if (!k_d || !v_d || layer < 0 || layer >= d.NL || B < 1 || B > d.maxB || T < 1 || pos0 < 0 || pos0 + T > d.S)
        return fail(h, LLM_EINVAL, "bad arguments");
    if ((rc = kv_reserve_uniform(h, B, 0, pos0 + T, false))) return rc;
    if ((rc = kv_upload(h))) return rc;
    return op_end(h, launch_kv_write(k_d, v_d, B, T, pos0, d.Hkv, d.hd, stream_len(h), kv_pages(h), d.dtype,
                                     layer_kc(h, layer), layer_vc(h, layer), h->stream));
}

int llm_op_attention(llm_t *h, int32_t layer, const void *q_d, int32_t B, int32_t T, int32_t pos0, void *out_d)
{
    int rc = op_begin(h);
    if (rc) return rc;
    const Dims &d = h->d;
    if (!q_d || !out_d || layer < 0 || layer >= d.NL || B < 1 || B > d.maxB || T < 1 || pos0 < 0 || pos0 + T > d.S)
        return fail(h, LLM_EINVAL, "bad arguments");
    if ((rc = kv_reserve_uniform(h, B, pos0 + T, pos0 + T, false))) return rc;
    if ((rc = kv_upload(h))) return rc;
    AttnArgs aa{};
    aa.q = q_d; aa.kcache = layer_kc(h, layer); aa.vcache = layer_vc(h, layer); aa.out = out_d;
    aa.B = B; aa.T = T; aa.H = d.H; aa.Hkv = d.Hkv; aa.hd = d.hd; aa.S = d.S;
    aa.Sb = stream_len(h);
    aa.pg = kv_pages(h);
    aa.pos_dev = nullptr; aa.pos_imm = pos0;
    hipError_t e;
    if (d.dtype == LLM_F32) e = launch_attn_f32(aa, h->stream);
    else if (T == 1) e = launch_attn_decode_f16(aa, h->stream);
    else if (pos0 == 0) e = launch_attn_prefill_f16(aa, h->stream);
    else return fail(h, LLM_EINVAL, "fp16 multi-token attention starts at position 0");
    return op_end(h, e);
}

int llm_op_layer(llm_t *h, int32_t layer, void *x_d, int32_t B, int32_t T, int32_t pos0)
{
    int rc = op_begin(h);
    if (rc) return rc;
    const Dims &d = h->d;
    if (!x_d || layer < 0 || layer >= d.NL || B < 1 || B > d.maxB || T < 1 || pos0 < 0 || (int64_t)pos0 + T > d.S)
        return fail(h, LLM_EINVAL, "bad arguments");
    if ((rc = ensure_ws(h, (int64_t)B * T))) return rc;
    if ((rc = kv_reserve_uniform(h, B, pos0, pos0 + T, false))) return rc;
    if ((rc = kv_upload(h))) return rc;
    const bool decode = T == 1 && pos0 >= 1;
    if (decode) {
        HIPC(h, launch_set_int(h->pos_dev, pos0, h->stream));
        h->dev_pos = pos0;
    }
    Pass ps = uniform_pass(B, T, decode ? h->pos_dev : nullptr, decode ? 0 : pos0);
    ps.x_given = true;
    const int64_t bytes = (int64_t)B * T * d.D * d.es;
    HIPC(h, hipMemcpyAsync(h->x, x_d, bytes, hipMemcpyDeviceToDevice, h->stream));
    LayerRun lr;
    lr.fused = fuse_norm(h, ps.M);
    lr.lay = act_layout(h, ps);
    const bool next = layer + 1 < d.NL;
    hipError_t e = layer_pass(h, ps, layer, lr, next, nullptr);
    // w2's split-K partials are added by the normalisation that opens the
    // next layer, as in a whole pass; its normalised rows are not used
    if (e == hipSuccess && lr.pend)
        e = norm_launch(h, lr, h->norm_w + (int64_t)(2 * (layer + 1)) * d.D * d.es, ps.M);
    if (e == hipSuccess) e = hipMemcpyAsync(x_d, h->x, bytes, hipMemcpyDeviceToDevice, h->stream);
    return op_end(h, e);
}

}  // extern "C"
