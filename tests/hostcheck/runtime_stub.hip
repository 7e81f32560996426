// Host-only stand-ins for the HIP runtime and the kernel launchers, so that
// the library's host logic runs without a GPU (under AddressSanitizer).
// Device memory is host memory and launches run nothing; the launchers that
// touch the KV cache check every cache address the kernel would compute.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include "../../llama_decoder_forward_amd/csrc/common.h"

static std::map<char *, size_t> g_alloc;
static bool in_alloc(const void *p, size_t bytes)
{
    const char *c = (const char *)p;
    auto it = g_alloc.upper_bound((char *)c);
    if (it == g_alloc.begin()) return false;
    --it;
    return c >= it->first && c + bytes <= it->first + it->second;
}
#define CHECK(p, n) do { if (!in_alloc((p), (n))) { fprintf(stderr, "OOB %s:%d %p +%zu\n", __FILE__, __LINE__, (const void*)(p), (size_t)(n)); abort(); } } while (0)

hipError_t hipMalloc(void **ptr, size_t size) { *ptr = calloc(1, size + 1); g_alloc[(char *)*ptr] = size; return hipSuccess; }
hipError_t hipHostMalloc(void **ptr, size_t size, unsigned int) { *ptr = malloc(size); return hipSuccess; }
hipError_t hipFree(void *p) { g_alloc.erase((char *)p); free(p); return hipSuccess; }
hipError_t hipHostFree(void *p) { free(p); return hipSuccess; }
hipError_t hipDeviceSynchronize(void) { return hipSuccess; }
hipError_t hipGetLastError(void) { return hipSuccess; }
const char *hipGetErrorString(hipError_t) { return "stub"; }
hipError_t hipStreamCreateWithFlags(hipStream_t *s, unsigned int) { *s = (hipStream_t)0x1; return hipSuccess; }
hipError_t hipStreamDestroy(hipStream_t) { return hipSuccess; }
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
hipError_t hipEventCreate(hipEvent_t *e) { *e = (hipEvent_t)malloc(8); return hipSuccess; }
hipError_t hipEventCreateWithFlags(hipEvent_t *e, unsigned) { *e = (hipEvent_t)malloc(8); return hipSuccess; }
hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipSuccess; }
hipError_t hipEventDestroy(hipEvent_t e) { free(e); return hipSuccess; }
hipError_t hipEventSynchronize(hipEvent_t) { return hipSuccess; }
hipError_t hipEventElapsedTime(float *ms, hipEvent_t, hipEvent_t) { *ms = 0.f; return hipSuccess; }
hipError_t hipGetDevice(int *d) { *d = 0; return hipSuccess; }
hipError_t hipDeviceGetAttribute(int *v, hipDeviceAttribute_t, int) { *v = 256; return hipSuccess; }
hipError_t hipMemGetInfo(size_t *fr, size_t *tot) { *tot = (size_t)1 << 36; *fr = *tot / 2; return hipSuccess; }
hipError_t hipMemcpyAsync(void *dst, const void *src, size_t n, hipMemcpyKind, hipStream_t) { memcpy(dst, src, n); return hipSuccess; }
hipError_t hipMemcpy2DAsync(void *dst, size_t dp, const void *src, size_t sp, size_t w, size_t hgt, hipMemcpyKind, hipStream_t)
{
    for (size_t r = 0; r < hgt; r++) memcpy((char *)dst + r * dp, (const char *)src + r * sp, w);
    return hipSuccess;
}
hipError_t hipStreamBeginCapture(hipStream_t, hipStreamCaptureMode) { return hipSuccess; }
hipError_t hipStreamEndCapture(hipStream_t, hipGraph_t *g) { *g = (hipGraph_t)malloc(8); return hipSuccess; }
hipError_t hipGraphDestroy(hipGraph_t g) { free(g); return hipSuccess; }
hipError_t hipGraphInstantiate(hipGraphExec_t *x, hipGraph_t, hipGraphNode_t *, char *, size_t) { *x = (hipGraphExec_t)malloc(8); return hipSuccess; }
hipError_t hipGraphLaunch(hipGraphExec_t, hipStream_t) { return hipSuccess; }
hipError_t hipGraphExecDestroy(hipGraphExec_t x) { free(x); return hipSuccess; }

bool skinny_can_normalise(int M, int K) { return M <= 2 && K <= 8192; }
hipError_t launch_gen_weights_f16(half_t *, int, int64_t, int64_t, uint64_t, int, int, int, int, int, bool, hipStream_t) { return hipSuccess; }
hipError_t launch_gen_weights_f32(float *, int, int64_t, int64_t, uint64_t, int, int, int, int, int, hipStream_t) { return hipSuccess; }
hipError_t launch_fill_f16(half_t *, int64_t, float, hipStream_t) { return hipSuccess; }
hipError_t launch_fill_f32(float *, int64_t, float, hipStream_t) { return hipSuccess; }
hipError_t launch_zero_bytes(void *d, int64_t n, hipStream_t) { CHECK(d, n); return hipSuccess; }
hipError_t launch_read_weights(const void *, int, int, int64_t, int64_t, int, int, int, int, int, int64_t, int64_t, void *, hipStream_t) { return hipSuccess; }
hipError_t launch_embed(const void *, const int32_t *, int64_t, int, int, const int *, int, const int *, const int2 *, int, int, void *, hipStream_t) { return hipSuccess; }
hipError_t launch_gather_rows(const void *, const int *, int, int, int, void *, hipStream_t) { return hipSuccess; }
hipError_t launch_rmsnorm(const void *, int64_t, const void *, int, int, float, int, void *, hipStream_t, int) { return hipSuccess; }
// the partial sums and the rows the residual form reads and writes
static int g_resid_norms = 0;  // normalisations that added handed-over partials
hipError_t launch_rmsnorm_resid(const float *part, int S, void *x, const void *, int M, int D, float, void *, hipStream_t, int)
{
    CHECK(part, (size_t)S * M * D * sizeof(float));
    CHECK(x, (size_t)M * D * 2);
    g_resid_norms++;
    return hipSuccess;
}
int hostcheck_resid_norms() { return g_resid_norms; }

// the cache addresses the KV write of rows (b, pos) touches
static int g_es = 2;
static void check_kv(const void *kc, const void *vc, const KvPages &pg, int Sb, int Hkv, int hd, int b, int pos)
{
    for (int kvh = 0; kvh < Hkv; kvh++) {
        if (pg.tab) CHECK(pg.tab + (int64_t)b * pg.ld + (pos >> pg.shift), 4);
        int off;
        int64_t st;
        if (pg.tab) {
            int blk = pg.tab[(int64_t)b * pg.ld + (pos >> pg.shift)];
            if (blk < 0) { fprintf(stderr, "empty table entry b=%d pos=%d\n", b, pos); abort(); }
        }
        // kv_stream is a device function; same arithmetic here
        if (pg.tab) { off = pos & ((1 << pg.shift) - 1); st = (int64_t)pg.tab[(int64_t)b * pg.ld + (pos >> pg.shift)] * Hkv + kvh; }
        else { off = pos; st = (int64_t)b * Hkv + kvh; }
        // fp16 K: the key's values are spread over its 32-position block (k16_offset)
        if (g_es == 2) CHECK((const char *)kc + k_offset(st, off & ~31, 0, Sb, hd) * g_es, (size_t)32 * hd * g_es);
        else CHECK((const char *)kc + k_offset(st, off, 0, Sb, hd) * g_es, (size_t)hd * g_es);
        const int64_t v0 = g_es == 2 ? v16_offset(st, off, 0, Sb, hd) : v32_offset(st, off, 0, Sb, hd);
        const int64_t v1 = g_es == 2 ? v16_offset(st, off, hd - 1, Sb, hd) : v32_offset(st, off, hd - 1, Sb, hd);
        CHECK((const char *)vc + v0 * g_es, g_es);
        CHECK((const char *)vc + v1 * g_es, g_es);
    }
}

static void check_qkv_ep(const GemmArgs &a)
{
    const Epilogue &ep = a.ep;
    if (ep.kind != EP_QKV) return;
    for (int m = 0; m < a.M; m++) {
        int b, pos;
        if (ep.rowmap) { b = ep.rowmap[m].x; pos = ep.rowmap[m].y; }
        else if (ep.pos_rows) { b = m; pos = ep.pos_rows[m]; }
        else { b = m / ep.T; pos = (ep.pos_dev ? *ep.pos_dev : ep.pos_imm) + m % ep.T; }
        check_kv(ep.kcache, ep.vcache, ep.pg, ep.S, ep.Hkv, ep.hd, b, pos);
    }
}
hipError_t launch_gemm_f16(const GemmArgs &a, hipStream_t)
{
    g_es = 2;
    check_qkv_ep(a);
    if (a.pending) {
        // as a split-K form would: residual products of fragment-major rows
        // leave four partial planes for the next normalisation launch
        *a.pending = 0;
        if (a.ep.kind == EP_RESID && a.ep.part && (a.x_lay == 1 || a.x_lay == 2)) {
            CHECK(a.ep.part, (size_t)4 * a.M * a.N * sizeof(float));
            *a.pending = 4;
        }
    }
    return hipSuccess;
}
hipError_t launch_linear_f32(const GemmArgs &a, hipStream_t) { g_es = 4; check_qkv_ep(a); return hipSuccess; }

static void check_attn(const AttnArgs &a, int es)
{
    g_es = es;
    for (int b = 0; b < a.B; b++) {
        int L;
        if (a.cu) L = a.cu[b + 1] - a.cu[b];
        else if (a.pos_rows) L = a.pos_rows[b] + 1;
        else L = (a.pos_dev ? *a.pos_dev : a.pos_imm) + a.T;
        for (int pos = 0; pos < L; pos++) check_kv(a.kcache, a.vcache, a.pg, a.Sb, a.Hkv, a.hd, b, pos);
    }
}
hipError_t launch_attn_decode_f16(const AttnArgs &a, hipStream_t) { check_attn(a, 2); return hipSuccess; }
hipError_t launch_attn_prefill_f16(const AttnArgs &a, hipStream_t) { check_attn(a, 2); return hipSuccess; }
hipError_t launch_attn_f32(const AttnArgs &a, hipStream_t) { check_attn(a, 4); return hipSuccess; }
hipError_t launch_kv_write(const void *, const void *, int B, int T, int pos0, int Hkv, int hd, int Sb, const KvPages &pg, int dtype, void *kc, void *vc, hipStream_t)
{
    g_es = dtype == 1 ? 2 : 4;
    for (int b = 0; b < B; b++)
        for (int t = 0; t < T; t++) check_kv(kc, vc, pg, Sb, Hkv, hd, b, pos0 + t);
    return hipSuccess;
}
hipError_t launch_argmax(const float *, int, int, int32_t *, int64_t, int, const int *, int32_t *, hipStream_t) { return hipSuccess; }
hipError_t launch_softmax_temp(const float *, int, int, float, float *, hipStream_t) { return hipSuccess; }
hipError_t launch_top_p(const float *, int, int, float, const float *, int32_t *, int64_t, int, const int *, int32_t *, hipStream_t) { return hipSuccess; }
hipError_t launch_sample_top_p(const float *, bool, float, int, int, float, const float *, int32_t *, int64_t, int, const int *, int32_t *, float *, hipStream_t) { return hipSuccess; }
hipError_t launch_set_int(int *d, int v, hipStream_t) { *d = v; return hipSuccess; }
const char *static_call_error() { return ""; }
hipError_t launch_inc_ints(int *d, int n, hipStream_t) { for (int i = 0; i < n; i++) d[i]++; return hipSuccess; }
hipError_t launch_set_tokens_rows(int32_t *, int64_t, int, const int *, const int32_t *, const uint8_t *, hipStream_t) { return hipSuccess; }
hipError_t launch_scatter_tokens(int32_t *, int64_t, int, const int2 *, const int32_t *, hipStream_t) { return hipSuccess; }
hipError_t launch_set_tokens(int32_t *, int64_t, int, int, const int32_t *, const uint8_t *, hipStream_t) { return hipSuccess; }

