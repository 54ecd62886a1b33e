// C-ABI layer of the gfx950 LoRA library: host-side argument checks,
// workspace planning and the kernel sequence of each entry point.  No entry
// point allocates device memory or synchronises the host.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "device_common.hpp"
#include "host_status.hpp"
#include "launch.hpp"
#include "lora_fused.h"

namespace lora {
size_t b1_lds_bytes(int C1, int r_lds);
size_t b2_lds_bytes(int C2, int r_lds);
}  // namespace lora

using namespace lora;

// ---------------------------------------------------------------------------
// Error reporting
// ---------------------------------------------------------------------------
static thread_local std::string g_last_error;

static lora_status fail(lora_status st, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

namespace lora {
lora_status host_fail(lora_status st, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}
}  // namespace lora

static lora_status hip_fail(hipError_t e, const char *what) {
    return fail(LORA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

extern "C" const char *lora_status_string(lora_status s) {
    // A C caller may pass any int; read it as one (a C++ load of an enum value
    // outside its enumerators' range is undefined).
    int v;
    std::memcpy(&v, &s, sizeof v);
    switch (v) {
    case LORA_OK: return "LORA_OK";
    case LORA_ERR_INVALID_ARG: return "LORA_ERR_INVALID_ARG";
    case LORA_ERR_UNSUPPORTED: return "LORA_ERR_UNSUPPORTED";
    case LORA_ERR_WORKSPACE: return "LORA_ERR_WORKSPACE";
    case LORA_ERR_HIP: return "LORA_ERR_HIP";
    }
    return "LORA_ERR_UNKNOWN";
}

extern "C" const char *lora_last_error_message(void) { return g_last_error.c_str(); }

// ---------------------------------------------------------------------------
// Kernel timing pool
// ---------------------------------------------------------------------------
namespace {
struct ProfSlot {
    const char *name;
    hipEvent_t ev0, ev1;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<ProfSlot> g_prof_pool;
size_t g_prof_used = 0;
}  // namespace

namespace lora {
int prof_begin(const char *name, hipStream_t stream) {
    if (!g_prof_on) return -1;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (g_prof_used >= g_prof_pool.size()) return -1;
    const int slot = (int)g_prof_used++;
    g_prof_pool[slot].name = name;
    (void)hipEventRecord(g_prof_pool[slot].ev0, stream);
    return slot;
}
void prof_end(int slot, hipStream_t stream) {
    if (slot < 0) return;
    (void)hipEventRecord(g_prof_pool[slot].ev1, stream);
}
}  // namespace lora

extern "C" lora_status lora_profiling_enable(int32_t enable, int32_t capacity) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    for (auto &s : g_prof_pool) {
        (void)hipEventDestroy(s.ev0);
        (void)hipEventDestroy(s.ev1);
    }
    g_prof_pool.clear();
    g_prof_used = 0;
    g_prof_on = false;
    if (!enable) return LORA_OK;
    if (capacity <= 0 || capacity > (1 << 20)) return fail(LORA_ERR_INVALID_ARG, "profiling capacity %d", capacity);
    g_prof_pool.resize((size_t)capacity);
    for (auto &s : g_prof_pool) {
        s.name = "";
        hipError_t e0 = hipEventCreate(&s.ev0);
        hipError_t e1 = hipEventCreate(&s.ev1);
        if (e0 != hipSuccess || e1 != hipSuccess) {
            g_prof_pool.clear();
            return hip_fail(e0 != hipSuccess ? e0 : e1, "hipEventCreate");
        }
    }
    g_prof_on = true;
    return LORA_OK;
}

extern "C" lora_status lora_profiling_reset(void) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof_used = 0;
    return LORA_OK;
}

extern "C" lora_status lora_profiling_query(const char *name_substring, int64_t *launches, double *total_ms) {
    if (!name_substring || !launches || !total_ms) return fail(LORA_ERR_INVALID_ARG, "NULL argument");
    std::lock_guard<std::mutex> lk(g_prof_mu);
    int64_t n = 0;
    double tot = 0.0;
    for (size_t i = 0; i < g_prof_used; ++i) {
        const ProfSlot &s = g_prof_pool[i];
        if (!std::strstr(s.name, name_substring)) continue;
        hipError_t e = hipEventSynchronize(s.ev1);
        if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
        float ms = 0.f;
        e = hipEventElapsedTime(&ms, s.ev0, s.ev1);
        if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
        ++n;
        tot += ms;
    }
    *launches = n;
    *total_ms = tot;
    return LORA_OK;
}

// ---------------------------------------------------------------------------
// Argument checks
// ---------------------------------------------------------------------------
static bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

#define REQUIRE(cond, ...)                                        \
    do {                                                          \
        if (!(cond)) return fail(LORA_ERR_INVALID_ARG, __VA_ARGS__); \
    } while (0)

static lora_status check_shape(int64_t m, int64_t k, int64_t n) {
    REQUIRE(m >= 0 && m < (1LL << 31), "m = %lld out of range [0, 2^31)", (long long)m);
    REQUIRE(k > 0 && k < (1LL << 31), "k = %lld out of range (0, 2^31)", (long long)k);
    REQUIRE(n > 0 && n < (1LL << 31), "n = %lld out of range (0, 2^31)", (long long)n);
    REQUIRE(k % 8 == 0, "k = %lld must be a multiple of 8", (long long)k);
    REQUIRE(n % 8 == 0, "n = %lld must be a multiple of 8", (long long)n);
    REQUIRE(m * k < (1LL << 46) && m * n < (1LL << 46), "tensor too large");
    return LORA_OK;
}

static lora_status check_rank(int32_t r) {
    REQUIRE(r >= 1 && r <= 256, "rank r = %d must be in [1, 256]", r);
    return LORA_OK;
}

// The GEMM epilogues and the dS/dB kernel address B (r x n bf16) and A
// (k x r bf16) with 32-bit byte offsets.
static lora_status check_b_size(int32_t r, int64_t k, int64_t n) {
    if ((int64_t)r * n * 2 >= (1LL << 31))
        return fail(LORA_ERR_UNSUPPORTED, "B of %d x %lld bf16 exceeds 2 GiB", r, (long long)n);
    if ((int64_t)r * k * 2 >= (1LL << 31))
        return fail(LORA_ERR_UNSUPPORTED, "A of %lld x %d bf16 exceeds 2 GiB", (long long)k, r);
    return LORA_OK;
}

static lora_status check_p(float p) {
    REQUIRE(p >= 0.0f && p < 1.0f, "dropout p = %g must be in [0, 1)", (double)p);
    return LORA_OK;
}

#define CHECK(x)                          \
    do {                                  \
        lora_status _st = (x);            \
        if (_st != LORA_OK) return _st;   \
    } while (0)

#define REQ_PTR(p, align) \
    REQUIRE((p) != nullptr && aligned((p), (align)), #p " must be non-NULL and %d-byte aligned", (int)(align))

// ---------------------------------------------------------------------------
// Workspace plans
// ---------------------------------------------------------------------------
namespace {
constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int cdiv(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

struct Carve {
    size_t off = 0;
    size_t take(size_t bytes) {
        size_t o = off;
        off = align_up(off + bytes);
        return o;
    }
};

struct FwdPlan {
    int RS;
    int chunk_cap_f1;  // grid size of F1 (upper bound on chunks)
    int chunk_cap_bwd;
    bool f1w;          // ranks 33..128: 64-row chunks sharing A, k in KS slices
    int KS, ksl;
    int s2_rp;  // > 0: F1 writes alpha*S as bf16 hi | lo rows of 2*s2_rp for the GEMM's extra K
    size_t off_spart, off_s2, off_t_f1, off_c_f1, off_t_bwd, off_c_bwd;
    size_t bytes;
};

// Ranks up to 32: F1 covers all of k inside each work-group (KS = 1).
// Ranks 33..128: 64-row chunks share A, and k is cut into KS slices
// (multiples of 128 columns) so the grid has about 512 work-groups (1024 for
// k >= 16384, where a slice's partial is under 2% of its X bytes and the
// second round of work-groups hides the first's latency); the slices'
// partials are added by a second launch.  Larger ranks: k in slices
// too (about 1024 work-groups), partials summed by a second pass.  KS depends
// on m and k only, so one segment of the mixed form slices as the single
// form does.
FwdPlan plan_fwd(int64_t m, int64_t k, int32_t RS, bool multi, int32_t nseg) {
    FwdPlan p{};
    p.RS = RS;
    p.chunk_cap_f1 = cdiv(m, kF1Rows) + (multi ? nseg : 0);
    p.chunk_cap_bwd = cdiv(m, kBwdRows) + (multi ? nseg : 0);
    const int rl = ((RS + 15) / 16) * 16;
    p.f1w = f1w_ok(rl, k);
    const int kslices = cdiv(k, kF1KSub);
    int KS = std::max(1, std::min(kslices, cdiv(p.f1w ? (k >= 16384 ? 1024 : 512) : 1024, std::max(1, cdiv(m, kF1Rows)))));
    if (!p.f1w && f1_streaming(rl, k)) KS = 1;
    const int per = cdiv(kslices, KS);
    p.ksl = per * kF1KSub;
    p.KS = cdiv(k, p.ksl);
    // single adapter, ranks 33..128: the up-projection runs as extra K
    // columns of the forward GEMM, fed by F1's split of alpha*S
    p.s2_rp = (!multi && p.f1w) ? rank_tiles(rl) * 32 : 0;
    const size_t part_w = p.f1w ? (size_t)16 * f1w_blocks(rl) : (size_t)RS;
    Carve c;
    p.off_spart = c.take(p.KS > 1 ? (size_t)p.KS * m * part_w * sizeof(float) : 0);
    p.off_s2 = c.take((size_t)m * 2 * p.s2_rp * sizeof(uint16_t));
    if (multi) {
        p.off_t_f1 = c.take((size_t)p.chunk_cap_f1 * sizeof(ChunkEntry));
        p.off_c_f1 = c.take(sizeof(int32_t));
        p.off_t_bwd = c.take((size_t)p.chunk_cap_bwd * sizeof(ChunkEntry));
        p.off_c_bwd = c.take(sizeof(int32_t));
    }
    p.bytes = c.off;
    return p;
}

struct BwdPlan {
    int RS;
    int rows2;  // rows per B2 work item (one dA partial each)
    int chunk_cap_bwd;
    int chunk_cap_f1;
    B1Shape b1;
    int C2;
    int ds_parts;  // dS partials written by B1 (one per column tile)
    bool b2w;      // the single-pass dA kernel (and its per-adapter sum launch)
    int items2;    // its grid rows of work items
    int dss_ld;    // > 0: B1's sum also writes split s*dS rows (dss_ld bf16 apart) for B2 and B3
    size_t off_ds, off_dspart, off_dbpart, off_dapart, off_t_f1, off_c_f1, off_t_bwd, off_c_bwd;
    size_t off_t_b1, off_c_b1, off_aditems, off_dss;
    size_t bytes;
};

BwdPlan plan_bwd(int64_t m, int64_t k, int64_t n, int32_t RS, bool multi, int32_t nseg, int32_t nad) {
    BwdPlan p{};
    p.RS = RS;
    const int rl = ((RS + 15) / 16) * 16;
    p.rows2 = b2_rows(m, k, rl);
    p.chunk_cap_bwd = cdiv(m, p.rows2) + (multi ? nseg : 0);
    p.chunk_cap_f1 = cdiv(m, kF1Rows) + (multi ? nseg : 0);
    p.b1 = b1_shape(m, n, rl, RS, multi, nseg);
    p.C2 = rl <= 128 ? 256 : 128;
    p.ds_parts = p.b1.CT;
    p.b2w = b2w_ok(rl, RS);
    p.items2 = multi ? p.chunk_cap_bwd : cdiv(m, p.rows2);
    p.dss_ld = p.b2w ? presplit_ld(rl) : 0;
    const int nct2 = cdiv(k, 256);
    Carve c;
    p.off_ds = c.take((size_t)m * RS * sizeof(float));
    p.off_dspart = c.take(p.ds_parts > 1 ? (size_t)p.ds_parts * m * RS * sizeof(float) : 0);
    p.off_dbpart = c.take((size_t)p.b1.slots * RS * n * sizeof(float));
    if (p.b2w)
        p.off_dapart = c.take((size_t)p.chunk_cap_bwd * nct2 * 256 * 16 * b2w_blocks(rl) * sizeof(float));
    else
        p.off_dapart = c.take((size_t)p.chunk_cap_bwd * k * RS * sizeof(float));
    p.off_aditems = c.take(multi ? (size_t)nad * sizeof(int32_t) : 0);
    p.off_dss = c.take((size_t)m * p.dss_ld * sizeof(uint16_t));
    if (multi) {
        p.off_t_f1 = c.take((size_t)p.chunk_cap_f1 * sizeof(ChunkEntry));
        p.off_c_f1 = c.take(sizeof(int32_t));
        p.off_t_bwd = c.take((size_t)p.chunk_cap_bwd * sizeof(ChunkEntry));
        p.off_c_bwd = c.take(sizeof(int32_t));
        p.off_t_b1 = c.take((size_t)p.b1.slots * sizeof(ChunkEntry));
        p.off_c_b1 = c.take(sizeof(int32_t));
    }
    p.bytes = c.off;
    return p;
}

char *ws_at(void *ws, size_t off) { return (char *)ws + off; }

AdapterSource single_source(const void *A, const void *B, void *dA, void *dB, int32_t r, float alpha, float p) {
    AdapterSource s{};
    s.A = A;
    s.B = B;
    s.dA = dA;
    s.dB = dB;
    s.r = r;
    s.alpha = alpha;
    s.p = p;
    s.table = nullptr;
    s.r_cap = r;
    return s;
}
}  // namespace

#define HIPCHK(call, what)                         \
    do {                                           \
        hipError_t _e = (call);                    \
        if (_e != hipSuccess) return hip_fail(_e, what); \
    } while (0)

// ---------------------------------------------------------------------------
// Single adapter
// ---------------------------------------------------------------------------
extern "C" size_t lora_linear_fwd_workspace_size(int64_t m, int64_t k, int64_t n, int32_t r) {
    (void)n;
    if (m < 0 || k <= 0 || r < 1) return 0;
    return plan_fwd(m, k, r, false, 0).bytes;
}

extern "C" size_t lora_linear_bwd_workspace_size(int64_t m, int64_t k, int64_t n, int32_t r) {
    if (m < 0 || k <= 0 || n <= 0 || r < 1) return 0;
    return plan_bwd(m, k, n, r, false, 0, 1).bytes;
}

extern "C" lora_status lora_linear_fwd(const void *X, const void *W, const void *A, const void *B,
                                       int64_t m, int64_t k, int64_t n, int32_t r, float alpha,
                                       float p, uint64_t seed, uint64_t offset, void *Y, float *S,
                                       uint32_t *keep_bits, void *workspace, size_t workspace_bytes,
                                       hipStream_t stream) {
    CHECK(check_shape(m, k, n));
    CHECK(check_rank(r));
    CHECK(check_p(p));
    CHECK(check_b_size(r, k, n));
    REQUIRE(offset % 8 == 0, "offset = %llu must be a multiple of 8", (unsigned long long)offset);
    REQ_PTR(W, 16);
    REQ_PTR(A, 2);
    REQ_PTR(B, 2);
    if (m == 0) return LORA_OK;  // nothing to compute; m-sized buffers may be NULL
    REQ_PTR(X, 16);
    REQ_PTR(Y, 16);
    REQ_PTR(S, 4);
    REQUIRE(keep_bits != nullptr || p == 0.0f, "keep_bits may be NULL only when p == 0");
    REQUIRE(aligned(keep_bits, 4), "keep_bits must be 4-byte aligned");
    const FwdPlan pl = plan_fwd(m, k, r, false, 0);
    if (workspace_bytes < pl.bytes)
        return fail(LORA_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, pl.bytes);
    if (pl.bytes) REQ_PTR(workspace, 16);

    AdapterSource src = single_source(A, B, nullptr, nullptr, r, alpha, p);
    float *spart = (float *)ws_at(workspace, pl.off_spart);
    // the extra-K form needs B's rows 16-byte aligned (n % 8 == 0 is checked above)
    uint16_t *s2 = (pl.s2_rp > 0 && aligned(B, 16)) ? (uint16_t *)ws_at(workspace, pl.off_s2) : nullptr;
    if (pl.f1w) {
        HIPCHK(launch_f1w(X, (int)m, (int)k, src, pl.chunk_cap_f1, seed, offset, keep_bits, S, r, spart, pl.KS,
                          pl.ksl, stream, s2, pl.s2_rp), "F1 launch");
    } else {
        float *sout = pl.KS > 1 ? spart : S;
        HIPCHK(launch_f1(X, (int)m, (int)k, src, pl.chunk_cap_f1, seed, offset, keep_bits, sout, r, pl.KS,
                         pl.ksl, stream), "F1 launch");
        if (pl.KS > 1)
            HIPCHK(launch_sum_partials(sout, pl.KS, (size_t)m * r, (size_t)m * r, S, "sum_s_partials", stream),
                   "S reduction launch");
    }
    if (s2)
        HIPCHK(launch_gemm_kext(X, W, Y, (int)m, (int)n, (int)k, s2, 2 * pl.s2_rp, B, r, stream), "F2 launch");
    else
        HIPCHK(launch_gemm(true, 1, X, W, Y, (int)m, (int)n, (int)k, S, r, nullptr, 0, src, stream), "F2 launch");
    return LORA_OK;
}

extern "C" lora_status lora_linear_fwd_concat(const void *X, const void *W, const void *A, const void *B,
                                              int64_t m, int64_t k, int64_t n, int32_t r, float alpha,
                                              void *Y, float *S, hipStream_t stream) {
    CHECK(check_shape(m, k, n));
    CHECK(check_rank(r));
    CHECK(check_b_size(r, k, n));
    REQ_PTR(W, 16);
    REQ_PTR(A, 2);
    REQ_PTR(B, 2);
    if (r != 8 && r != 16)
        return fail(LORA_ERR_UNSUPPORTED, "the concatenated forward takes r = 8 or 16 (r = %d)", r);
    if (!aligned(A, 16) || !aligned(B, 16))
        return fail(LORA_ERR_UNSUPPORTED, "the concatenated forward needs A and B 16-byte aligned");
    if (m == 0) return LORA_OK;
    REQ_PTR(X, 16);
    REQ_PTR(Y, 16);
    REQ_PTR(S, 4);
    if (!aligned(S, 16)) return fail(LORA_ERR_UNSUPPORTED, "the concatenated forward needs S 16-byte aligned");
    HIPCHK(launch_gemm_cat(X, W, A, B, Y, S, (int)m, (int)n, (int)k, r, alpha, stream), "concatenated F2 launch");
    return LORA_OK;
}

extern "C" lora_status lora_linear_bwd(const void *dY, const void *X, const void *W, const void *A,
                                       const void *B, const float *S, const uint32_t *keep_bits,
                                       int64_t m, int64_t k, int64_t n, int32_t r, float alpha,
                                       float p, void *dX, void *dA, void *dB, void *workspace,
                                       size_t workspace_bytes, hipStream_t stream) {
    CHECK(check_shape(m, k, n));
    CHECK(check_rank(r));
    CHECK(check_p(p));
    CHECK(check_b_size(r, k, n));
    REQ_PTR(W, 16);
    REQ_PTR(A, 2);
    REQ_PTR(B, 2);
    REQ_PTR(dA, 2);
    REQ_PTR(dB, 2);
    if (m > 0) {  // m-sized buffers may be NULL when m == 0 (then dA = dB = 0)
        REQ_PTR(dY, 16);
        REQ_PTR(X, 16);
        REQ_PTR(S, 4);
        REQUIRE(dX == nullptr || aligned(dX, 16), "dX must be 16-byte aligned (or NULL: no input gradient)");
        REQUIRE(keep_bits != nullptr || p == 0.0f, "keep_bits may be NULL only when p == 0");
        REQUIRE(aligned(keep_bits, 4), "keep_bits must be 4-byte aligned");
    }
    const BwdPlan pl = plan_bwd(m, k, n, r, false, 0, 1);
    if (workspace_bytes < pl.bytes)
        return fail(LORA_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, pl.bytes);
    if (pl.bytes) REQ_PTR(workspace, 16);

    AdapterSource src = single_source(A, B, dA, dB, r, alpha, p);
    float *dS = (float *)ws_at(workspace, pl.off_ds);
    float *dSpart = pl.ds_parts > 1 ? (float *)ws_at(workspace, pl.off_dspart) : dS;
    float *dBpart = (float *)ws_at(workspace, pl.off_dbpart);
    float *dApart = (float *)ws_at(workspace, pl.off_dapart);
    uint16_t *dss = pl.dss_ld > 0 ? (uint16_t *)ws_at(workspace, pl.off_dss) : nullptr;
    const int chunks = pl.chunk_cap_bwd;
    if (m > 0) HIPCHK(launch_b1(dY, S, (int)m, (int)n, r, src, pl.b1, dSpart, dBpart, stream), "B1 launch");
    HIPCHK(launch_b1_reduce(dSpart, m > 0 ? pl.ds_parts : 1, dS, dBpart, (int)m, (int)n, r, src, pl.b1.rows,
                            pl.b1.slots, stream, dss, pl.dss_ld),
           "dS/dB reduction launch");
    if (pl.b2w) {
        HIPCHK(launch_b2w(X, p == 0.0f ? nullptr : keep_bits, dS, (int)m, (int)k, r, pl.rows2, src, pl.items2,
                          dApart, nullptr, stream, dss, pl.dss_ld), "B2 launch");
    } else {
        if (m > 0)
            HIPCHK(launch_b2(X, p == 0.0f ? nullptr : keep_bits, dS, (int)m, (int)k, r, pl.rows2, src, chunks,
                             pl.C2, dApart, stream), "B2 launch");
        HIPCHK(launch_grad_reduce(1, dApart, (int)m, (int)k, (int)n, r, src, pl.rows2, chunks, stream),
               "dA reduction launch");
    }
    if (m > 0 && dX != nullptr)
        HIPCHK(launch_gemm(false, 2, dY, W, dX, (int)m, (int)k, (int)n, dS, r, p == 0.0f ? nullptr : keep_bits,
                           (int)((k + 31) / 32), src, stream, dss, pl.dss_ld), "B3 launch");
    return LORA_OK;
}

// ---------------------------------------------------------------------------
// Multi adapter
// ---------------------------------------------------------------------------
static lora_status check_multi(const lora_adapter *adapters, int32_t num_adapters, const int64_t *seg_off,
                               const int32_t *seg_adapter, int32_t num_segments, int32_t r_max) {
    REQUIRE(adapters != nullptr && aligned(adapters, 8), "adapters must be a non-NULL 8-byte aligned device array");
    REQUIRE(num_adapters >= 1 && num_adapters <= (1 << 20), "num_adapters = %d out of range", num_adapters);
    REQUIRE(seg_off != nullptr && aligned(seg_off, 8), "seg_off must be non-NULL and 8-byte aligned");
    REQUIRE(seg_adapter != nullptr && aligned(seg_adapter, 4), "seg_adapter must be non-NULL and 4-byte aligned");
    REQUIRE(num_segments >= 1 && num_segments <= (1 << 24), "num_segments = %d out of range", num_segments);
    CHECK(check_rank(r_max));
    return LORA_OK;
}

extern "C" size_t multi_lora_fwd_workspace_size(int64_t m, int64_t k, int64_t n, int32_t r_max,
                                                int32_t num_adapters, int32_t num_segments) {
    (void)n;
    (void)num_adapters;
    if (m < 0 || k <= 0 || r_max < 1 || num_segments < 0) return 0;
    return plan_fwd(m, k, r_max, true, num_segments).bytes;
}

extern "C" size_t multi_lora_bwd_workspace_size(int64_t m, int64_t k, int64_t n, int32_t r_max,
                                                int32_t num_adapters, int32_t num_segments) {
    if (m < 0 || k <= 0 || n <= 0 || r_max < 1 || num_segments < 0 || num_adapters < 1) return 0;
    return plan_bwd(m, k, n, r_max, true, num_segments, num_adapters).bytes;
}

static AdapterSource multi_source(const lora_adapter *adapters, int32_t nad, const int64_t *seg_off,
                                  const int32_t *seg_adapter, int32_t nseg, int32_t r_max) {
    AdapterSource s{};
    s.table = adapters;
    s.num_adapters = nad;
    s.r_cap = r_max;
    s.seg_off = seg_off;
    s.seg_adapter = seg_adapter;
    s.num_segments = nseg;
    s.r = r_max;
    return s;
}

extern "C" lora_status multi_lora_linear_fwd(const void *X, const void *W, const lora_adapter *adapters,
                                             int32_t num_adapters, const int64_t *seg_off,
                                             const int32_t *seg_adapter, int32_t num_segments, int64_t m,
                                             int64_t k, int64_t n, int32_t r_max, uint64_t seed,
                                             uint64_t offset, void *Y, float *S, uint32_t *keep_bits,
                                             void *workspace, size_t workspace_bytes, hipStream_t stream) {
    CHECK(check_shape(m, k, n));
    CHECK(check_multi(adapters, num_adapters, seg_off, seg_adapter, num_segments, r_max));
    CHECK(check_b_size(r_max, k, n));
    REQUIRE(offset % 8 == 0, "offset = %llu must be a multiple of 8", (unsigned long long)offset);
    REQ_PTR(W, 16);
    if (m == 0) return LORA_OK;
    REQ_PTR(X, 16);
    REQ_PTR(Y, 16);
    REQ_PTR(S, 4);
    REQ_PTR(keep_bits, 4);
    const FwdPlan pl = plan_fwd(m, k, r_max, true, num_segments);
    if (workspace_bytes < pl.bytes)
        return fail(LORA_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, pl.bytes);
    REQ_PTR(workspace, 16);

    AdapterSource src = multi_source(adapters, num_adapters, seg_off, seg_adapter, num_segments, r_max);
    src.chunks_f1 = (const ChunkEntry *)ws_at(workspace, pl.off_t_f1);
    src.count_f1 = (const int32_t *)ws_at(workspace, pl.off_c_f1);
    src.chunks_bwd = (const ChunkEntry *)ws_at(workspace, pl.off_t_bwd);
    src.count_bwd = (const int32_t *)ws_at(workspace, pl.off_c_bwd);
    HIPCHK(launch_router(seg_off, seg_adapter, num_segments, (int)m, adapters, num_adapters, r_max,
                         (ChunkEntry *)src.chunks_f1, (int32_t *)src.count_f1, pl.chunk_cap_f1,
                         (ChunkEntry *)src.chunks_bwd, (int32_t *)src.count_bwd, kBwdRows, pl.chunk_cap_bwd,
                         nullptr, nullptr, 0, 0, stream),
           "router launch");
    float *spart = (float *)ws_at(workspace, pl.off_spart);
    if (pl.f1w) {
        HIPCHK(launch_f1w(X, (int)m, (int)k, src, pl.chunk_cap_f1, seed, offset, keep_bits, S, r_max, spart,
                          pl.KS, pl.ksl, stream), "F1 launch");
    } else {
        float *sout = pl.KS > 1 ? spart : S;
        HIPCHK(launch_f1(X, (int)m, (int)k, src, pl.chunk_cap_f1, seed, offset, keep_bits, sout, r_max, pl.KS,
                         pl.ksl, stream), "F1 launch");
        if (pl.KS > 1)
            HIPCHK(launch_sum_partials(sout, pl.KS, (size_t)m * r_max, (size_t)m * r_max, S, "sum_s_partials",
                                       stream), "S reduction launch");
    }
    HIPCHK(launch_gemm(true, 1, X, W, Y, (int)m, (int)n, (int)k, S, r_max, nullptr, 0, src, stream), "F2 launch");
    return LORA_OK;
}

extern "C" lora_status multi_lora_linear_bwd(const void *dY, const void *X, const void *W,
                                             const lora_adapter *adapters, int32_t num_adapters,
                                             const int64_t *seg_off, const int32_t *seg_adapter,
                                             int32_t num_segments, const float *S, const uint32_t *keep_bits,
                                             int64_t m, int64_t k, int64_t n, int32_t r_max, void *dX,
                                             void *workspace, size_t workspace_bytes, hipStream_t stream) {
    CHECK(check_shape(m, k, n));
    CHECK(check_multi(adapters, num_adapters, seg_off, seg_adapter, num_segments, r_max));
    CHECK(check_b_size(r_max, k, n));
    REQ_PTR(W, 16);
    if (m > 0) {
        REQ_PTR(dY, 16);
        REQ_PTR(X, 16);
        REQ_PTR(S, 4);
        REQ_PTR(keep_bits, 4);
        REQUIRE(dX == nullptr || aligned(dX, 16), "dX must be 16-byte aligned (or NULL: no input gradient)");
    }
    const BwdPlan pl = plan_bwd(m, k, n, r_max, true, num_segments, num_adapters);
    if (workspace_bytes < pl.bytes)
        return fail(LORA_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, pl.bytes);
    REQ_PTR(workspace, 16);

    AdapterSource src = multi_source(adapters, num_adapters, seg_off, seg_adapter, num_segments, r_max);
    src.chunks_f1 = (const ChunkEntry *)ws_at(workspace, pl.off_t_f1);
    src.count_f1 = (const int32_t *)ws_at(workspace, pl.off_c_f1);
    src.chunks_bwd = (const ChunkEntry *)ws_at(workspace, pl.off_t_bwd);
    src.count_bwd = (const int32_t *)ws_at(workspace, pl.off_c_bwd);
    src.chunks_b1 = (const ChunkEntry *)ws_at(workspace, pl.off_t_b1);
    src.count_b1 = (const int32_t *)ws_at(workspace, pl.off_c_b1);
    int32_t *aditems = (int32_t *)ws_at(workspace, pl.off_aditems);
    HIPCHK(launch_router(seg_off, seg_adapter, num_segments, (int)m, adapters, num_adapters, r_max,
                         (ChunkEntry *)src.chunks_f1, (int32_t *)src.count_f1, pl.chunk_cap_f1,
                         (ChunkEntry *)src.chunks_bwd, (int32_t *)src.count_bwd, pl.rows2, pl.chunk_cap_bwd,
                         (ChunkEntry *)src.chunks_b1, (int32_t *)src.count_b1, pl.b1.rows, pl.b1.slots, stream,
                         aditems),
           "router launch");
    float *dS = (float *)ws_at(workspace, pl.off_ds);
    float *dSpart = pl.ds_parts > 1 ? (float *)ws_at(workspace, pl.off_dspart) : dS;
    float *dBpart = (float *)ws_at(workspace, pl.off_dbpart);
    float *dApart = (float *)ws_at(workspace, pl.off_dapart);
    uint16_t *dss = pl.dss_ld > 0 ? (uint16_t *)ws_at(workspace, pl.off_dss) : nullptr;
    const int chunks = pl.chunk_cap_bwd;
    if (m > 0) HIPCHK(launch_b1(dY, S, (int)m, (int)n, r_max, src, pl.b1, dSpart, dBpart, stream), "B1 launch");
    HIPCHK(launch_b1_reduce(dSpart, m > 0 ? pl.ds_parts : 1, dS, dBpart, (int)m, (int)n, r_max, src, pl.b1.rows,
                            pl.b1.slots, stream, dss, pl.dss_ld),
           "dS/dB reduction launch");
    if (pl.b2w) {
        HIPCHK(launch_b2w(X, keep_bits, dS, (int)m, (int)k, r_max, pl.rows2, src, pl.items2, dApart, aditems,
                          stream, dss, pl.dss_ld), "B2 launch");
    } else {
        if (m > 0)
            HIPCHK(launch_b2(X, keep_bits, dS, (int)m, (int)k, r_max, pl.rows2, src, chunks, pl.C2, dApart, stream),
                   "B2 launch");
        HIPCHK(launch_grad_reduce(1, dApart, (int)m, (int)k, (int)n, r_max, src, pl.rows2, chunks, stream),
               "dA reduction launch");
    }
    if (m > 0 && dX != nullptr)
        HIPCHK(launch_gemm(false, 2, dY, W, dX, (int)m, (int)k, (int)n, dS, r_max, keep_bits, (int)((k + 31) / 32),
                           src, stream, dss, pl.dss_ld), "B3 launch");
    return LORA_OK;
}

extern "C" lora_status multi_lora_check_segments(const int64_t *seg_off_host, const int32_t *seg_adapter_host,
                                                 int32_t num_segments, int64_t m, const int32_t *adapter_r_host,
                                                 int32_t num_adapters, int32_t r_max) {
    REQUIRE(seg_off_host && seg_adapter_host && adapter_r_host, "NULL host array");
    REQUIRE(num_segments >= 1, "num_segments = %d must be >= 1", num_segments);
    REQUIRE(num_adapters >= 1, "num_adapters = %d must be >= 1", num_adapters);
    REQUIRE(seg_off_host[0] == 0, "seg_off[0] = %lld must be 0", (long long)seg_off_host[0]);
    REQUIRE(seg_off_host[num_segments] == m, "seg_off[last] = %lld must equal m = %lld",
            (long long)seg_off_host[num_segments], (long long)m);
    for (int32_t s = 0; s < num_segments; ++s) {
        REQUIRE(seg_off_host[s + 1] >= seg_off_host[s], "segment %d has negative length", s);
        REQUIRE(seg_adapter_host[s] >= 0 && seg_adapter_host[s] < num_adapters,
                "segment %d uses adapter %d outside [0, %d)", s, seg_adapter_host[s], num_adapters);
    }
    for (int32_t a = 0; a < num_adapters; ++a)
        REQUIRE(adapter_r_host[a] >= 1 && adapter_r_host[a] <= r_max, "adapter %d rank %d outside [1, r_max = %d]",
                a, adapter_r_host[a], r_max);
    return LORA_OK;
}

// ---------------------------------------------------------------------------
// DoRA norm
// ---------------------------------------------------------------------------
extern "C" size_t lora_dora_norm_workspace_size(int64_t k, int64_t n, int32_t r) {
    if (k <= 0 || n <= 0 || k >= (1LL << 31) || n >= (1LL << 31)) return 0;
    const DoraPlan pl = dora_plan(k, n, r);
    return (size_t)pl.splits * (size_t)n * sizeof(float);
}

extern "C" lora_status lora_dora_norm(const void *W, const void *A, const void *B, int64_t k, int64_t n,
                                      int32_t r, float alpha, float *norm, void *workspace,
                                      size_t workspace_bytes, hipStream_t stream) {
    REQUIRE(k > 0 && k < (1LL << 31), "k = %lld out of range (0, 2^31)", (long long)k);
    REQUIRE(n > 0 && n < (1LL << 31), "n = %lld out of range (0, 2^31)", (long long)n);
    REQUIRE(n % 8 == 0, "n = %lld must be a multiple of 8", (long long)n);
    CHECK(check_rank(r));
    REQ_PTR(W, 16);
    REQ_PTR(A, 16);
    REQ_PTR(B, 16);
    REQ_PTR(norm, 4);
    if ((int64_t)(r + 32) * n * 2 >= (1LL << 31) || k * (int64_t)r * 2 >= (1LL << 31))
        return fail(LORA_ERR_UNSUPPORTED, "A or B exceeds 2 GiB");
    const DoraPlan pl = dora_plan(k, n, r);
    const size_t need = (size_t)pl.splits * (size_t)n * sizeof(float);
    if (workspace_bytes < need)
        return fail(LORA_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", workspace_bytes, need);
    REQ_PTR(workspace, 16);
    HIPCHK(launch_dora_norm(W, A, B, (int)k, (int)n, r, alpha, pl, (float *)workspace, norm, stream),
           "DoRA norm launch");
    return LORA_OK;
}

// ---------------------------------------------------------------------------
// Pieces
// ---------------------------------------------------------------------------
extern "C" lora_status lora_dropout_mask(uint64_t seed, uint64_t offset, int64_t m, int64_t k, float p,
                                         uint32_t *keep_bits, hipStream_t stream) {
    REQUIRE(m >= 0 && m < (1LL << 31), "m out of range");
    REQUIRE(k > 0 && k < (1LL << 31) && k % 8 == 0, "k must be a positive multiple of 8");
    CHECK(check_p(p));
    REQUIRE(offset % 8 == 0, "offset must be a multiple of 8");
    REQ_PTR(keep_bits, 4);
    HIPCHK(launch_mask(seed, offset, (int)m, (int)k, p, keep_bits, stream), "mask launch");
    return LORA_OK;
}

extern "C" lora_status lora_frozen_fwd(const void *X, const void *W, int64_t m, int64_t k, int64_t n, void *Y,
                                       hipStream_t stream) {
    CHECK(check_shape(m, k, n));
    REQ_PTR(X, 16);
    REQ_PTR(W, 16);
    REQ_PTR(Y, 16);
    AdapterSource src{};
    HIPCHK(launch_gemm(true, 0, X, W, Y, (int)m, (int)n, (int)k, nullptr, 0, nullptr, 0, src, stream),
           "frozen fwd launch");
    return LORA_OK;
}

extern "C" lora_status lora_frozen_bwd(const void *dY, const void *W, int64_t m, int64_t k, int64_t n, void *dX,
                                       hipStream_t stream) {
    CHECK(check_shape(m, k, n));
    REQ_PTR(dY, 16);
    REQ_PTR(W, 16);
    REQ_PTR(dX, 16);
    AdapterSource src{};
    HIPCHK(launch_gemm(false, 0, dY, W, dX, (int)m, (int)k, (int)n, nullptr, 0, nullptr, 0, src, stream),
           "frozen bwd launch");
    return LORA_OK;
}

// ---------------------------------------------------------------------------
// Backward without a workspace argument, for callers that cannot allocate
// device memory (code under graph capture, tight loops, harnesses that forbid
// it).  Its scratch is a file-scope device array of kScratchBytes: every GPU
// the library runs on holds one copy until the process ends.  The array's
// name is a host-side stand-in; its device address comes from
// hipGetSymbolAddress, once per device, and only that address is passed on.
// ---------------------------------------------------------------------------
namespace {
constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr int kScratchDevices = 64;
}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
std::mutex g_scratch_mu;
void *g_scratch_ptr[kScratchDevices] = {};
}  // namespace

static lora_status scratch_of_current_device(void **out) {
    int dev = -1;
    HIPCHK(hipGetDevice(&dev), "hipGetDevice");
    if (dev < 0 || dev >= kScratchDevices)
        return fail(LORA_ERR_UNSUPPORTED, "device %d: the static scratch serves devices 0..%d", dev,
                    kScratchDevices - 1);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void *p = nullptr;
        HIPCHK(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
        if (p == nullptr) return fail(LORA_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return LORA_OK;
}

extern "C" size_t lora_linear_bwd_noalloc_max_scratch(void) { return kScratchBytes; }

extern "C" lora_status lora_linear_bwd_noalloc(const void *dY, const void *X, const void *W, const void *A,
                                               const void *B, const float *S, const uint32_t *keep_bits,
                                               int64_t m, int64_t k, int64_t n, int32_t r, float alpha, float p,
                                               void *dX, void *dA, void *dB, hipStream_t stream) {
    CHECK(check_shape(m, k, n));
    CHECK(check_rank(r));
    const size_t need = plan_bwd(m, k, n, r, false, 0, 1).bytes;
    if (need > kScratchBytes)
        return fail(LORA_ERR_UNSUPPORTED,
                    "shape m=%lld k=%lld n=%lld r=%d needs %zu bytes of scratch; the static scratch holds %zu "
                    "(use lora_linear_bwd with a workspace)",
                    (long long)m, (long long)k, (long long)n, r, need, kScratchBytes);
    void *ws = nullptr;
    CHECK(scratch_of_current_device(&ws));
    return lora_linear_bwd(dY, X, W, A, B, S, keep_bits, m, k, n, r, alpha, p, dX, dA, dB, ws, kScratchBytes,
                           stream);
}
