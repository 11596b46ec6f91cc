// api.cpp -- the extern "C" boundary declared in include/ptq1.h.
//
// Every entry point validates all arguments on the host before anything is
// enqueued (null pointers, shapes, alignment, overlap, int64 overflow,
// workspace size) and names the refused argument in ptq1_last_error().
// Conventions follow "Why I Am Building Another Inference Engine", Level 4:
// the C header is the ABI, every call returns a status the caller checks,
// and sizes are computed with checked arithmetic.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/ptq1.h"
#include "ptq1_geometry.h"
#include "ptq1_launch.h"

static_assert(PTQ1_BLOCK_WEIGHTS == ptq1::kBlockWeights, "public header and geometry agree");
static_assert(PTQ1_TRIT_BYTES == ptq1::kTritBytes, "public header and geometry agree");
static_assert(PTQ1_BLOCK_BYTES == ptq1::kBlockBytes, "public header and geometry agree");
static_assert(PTQ1_HADAMARD == ptq1::kHadamard, "public header and geometry agree");
static_assert(PTQ1_TILE_ROWS == ptq1::kTileRows, "public header and geometry agree");
static_assert(PTQ1_TILE_BLOCKS == ptq1::kTileBlocks, "public header and geometry agree");

namespace {

thread_local std::string g_last_error;

ptq1_status fail(ptq1_status s, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

ptq1_status ok()
{
    g_last_error.clear();
    return PTQ1_OK;
}

ptq1_status hip_status(hipError_t e, const char *what)
{
    if (e == hipSuccess) return ok();
    return fail(PTQ1_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool mul_ok(int64_t a, int64_t b, int64_t *out) { return !__builtin_mul_overflow(a, b, out); }

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// [a, a + na) and [b, b + nb) share a byte
bool overlaps(const void *a, int64_t na, const void *b, int64_t nb)
{
    if (na <= 0 || nb <= 0 || a == nullptr || b == nullptr) return false;
    const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
    return pa < pb + static_cast<uintptr_t>(nb) && pb < pa + static_cast<uintptr_t>(na);
}

constexpr uintptr_t kAlign = 16;
constexpr size_t kWsAlign = 256;
constexpr int64_t kMaxGemmM = 65536;
constexpr int64_t kMaxGridX = 2147483647;
constexpr int64_t kMaxGridY = 65535;
// Decode calls: rows per matrix (keeps the matvec grid's second dimension,
// chunks of 32-row groups, far below its limit).
constexpr int64_t kMaxLutRows = int64_t{1} << 20;

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Packed bytes with every check; -1 on a bad shape or overflow.
int64_t packed_bytes(int64_t n, int64_t k)
{
    if (n < 0 || k < 0 || k % ptq1::kBlockWeights != 0) return -1;
    int64_t nb_bytes, total;
    if (!mul_ok(k / ptq1::kBlockWeights, ptq1::kBlockBytes, &nb_bytes)) return -1;
    if (!mul_ok(n, nb_bytes, &total)) return -1;
    return total;
}

// Tiled-layout bytes with every check; -1 on a bad shape or overflow.
int64_t tiled_bytes(int64_t n, int64_t k)
{
    if (n < 0 || k < 0 || k % ptq1::kBlockWeights != 0) return -1;
    const int64_t bands = n / ptq1::kTileRows + (n % ptq1::kTileRows != 0);
    const int64_t nb = k / ptq1::kBlockWeights;
    const int64_t tiles_k = nb / ptq1::kTileBlocks + (nb % ptq1::kTileBlocks != 0);
    int64_t tiles, total;
    if (!mul_ok(bands, tiles_k, &tiles)) return -1;
    if (!mul_ok(tiles, ptq1::kTileBytes, &total)) return -1;
    return total;
}

// The lookup-table matvec addresses a tiled matrix with 32-bit offsets.
constexpr int64_t kMaxLutMatrixBytes = int64_t{1} << 31;

// Shared validation of a packed (tiled = false) or tiled matrix argument.
ptq1_status check_matrix(const uint8_t *blocks, const char *name, int64_t n, int64_t k,
                         bool need_1024, int64_t *bytes, bool tiled = false)
{
    if (n < 0) return fail(PTQ1_ERR_SHAPE, "%s: n = %lld is negative", name, (long long)n);
    if (k < 0) return fail(PTQ1_ERR_SHAPE, "%s: k = %lld is negative", name, (long long)k);
    if (k % ptq1::kBlockWeights != 0)
        return fail(PTQ1_ERR_SHAPE, "%s: k = %lld is not a multiple of %d", name, (long long)k,
                    ptq1::kBlockWeights);
    if (need_1024 && k % ptq1::kHadamard != 0)
        return fail(PTQ1_ERR_SHAPE, "%s: k = %lld is not a multiple of %d (rotation chunks)", name,
                    (long long)k, ptq1::kHadamard);
    const int64_t b = tiled ? tiled_bytes(n, k) : packed_bytes(n, k);
    if (b < 0 || packed_bytes(n, k) < 0)
        return fail(PTQ1_ERR_OVERFLOW, "%s: size of [%lld][%lld] overflows", name, (long long)n, (long long)k);
    if (b > 0 && blocks == nullptr) return fail(PTQ1_ERR_NULL, "%s is NULL", name);
    if (b > 0 && !aligned(blocks, kAlign)) return fail(PTQ1_ERR_ALIGN, "%s is not 16-byte aligned", name);
    *bytes = b;
    return PTQ1_OK;
}

// PQ2_0 sizes (34-byte blocks; tiles of 32 rows x 2 blocks, 2176 bytes):
// -1 on a bad shape or overflow.
int64_t pq2_packed(int64_t n, int64_t k)
{
    if (n < 0 || k < 0 || k % ptq1::kBlockWeights != 0) return -1;
    int64_t nb_bytes, total;
    if (!mul_ok(k / ptq1::kBlockWeights, ptq1::kPq2BlockBytes, &nb_bytes)) return -1;
    if (!mul_ok(n, nb_bytes, &total)) return -1;
    return total;
}

int64_t pq2_tiled(int64_t n, int64_t k)
{
    if (pq2_packed(n, k) < 0) return -1;
    const int64_t bands = n / ptq1::kTileRows + (n % ptq1::kTileRows != 0);
    const int64_t nb = k / ptq1::kBlockWeights;
    const int64_t tiles_k = nb / ptq1::kTileBlocks + (nb % ptq1::kTileBlocks != 0);
    int64_t tiles, total;
    if (!mul_ok(bands, tiles_k, &tiles)) return -1;
    if (!mul_ok(tiles, ptq1::kPq2TileBytes, &total)) return -1;
    return total;
}

ptq1_status check_pq2(const uint8_t *blocks, const char *name, int64_t n, int64_t k, bool need_1024,
                      int64_t *bytes, bool tiled)
{
    if (n < 0) return fail(PTQ1_ERR_SHAPE, "%s: n = %lld is negative", name, (long long)n);
    if (k < 0) return fail(PTQ1_ERR_SHAPE, "%s: k = %lld is negative", name, (long long)k);
    if (k % ptq1::kBlockWeights != 0)
        return fail(PTQ1_ERR_SHAPE, "%s: k = %lld is not a multiple of %d", name, (long long)k,
                    ptq1::kBlockWeights);
    if (need_1024 && k % ptq1::kHadamard != 0)
        return fail(PTQ1_ERR_SHAPE, "%s: k = %lld is not a multiple of %d (rotation chunks)", name,
                    (long long)k, ptq1::kHadamard);
    const int64_t b = tiled ? pq2_tiled(n, k) : pq2_packed(n, k);
    if (b < 0) return fail(PTQ1_ERR_OVERFLOW, "%s: size of [%lld][%lld] overflows", name, (long long)n, (long long)k);
    if (b > 0 && blocks == nullptr) return fail(PTQ1_ERR_NULL, "%s is NULL", name);
    if (b > 0 && !aligned(blocks, kAlign)) return fail(PTQ1_ERR_ALIGN, "%s is not 16-byte aligned", name);
    *bytes = b;
    return PTQ1_OK;
}

ptq1_status check_floats(const void *p, const char *name, int64_t count, int64_t *bytes)
{
    int64_t b;
    if (count < 0) return fail(PTQ1_ERR_SHAPE, "%s: negative element count", name);
    if (!mul_ok(count, 4, &b)) return fail(PTQ1_ERR_OVERFLOW, "%s: byte size overflows", name);
    if (count > 0 && p == nullptr) return fail(PTQ1_ERR_NULL, "%s is NULL", name);
    if (count > 0 && !aligned(p, kAlign)) return fail(PTQ1_ERR_ALIGN, "%s is not 16-byte aligned", name);
    *bytes = b;
    return PTQ1_OK;
}

ptq1_status check_signs(const float *signs, bool required)
{
    if (signs == nullptr) {
        if (required) return fail(PTQ1_ERR_NULL, "signs1024 is NULL");
        return PTQ1_OK;
    }
    if (!aligned(signs, kAlign)) return fail(PTQ1_ERR_ALIGN, "signs1024 is not 16-byte aligned");
    return PTQ1_OK;
}

ptq1_status check_ws(const void *ws, size_t ws_bytes, size_t need, const char *fn)
{
    if (need == 0) return PTQ1_OK;
    if (ws == nullptr) return fail(PTQ1_ERR_WORKSPACE, "%s: ws is NULL (%zu bytes needed)", fn, need);
    if (ws_bytes < need)
        return fail(PTQ1_ERR_WORKSPACE, "%s: ws_bytes = %zu < %zu needed", fn, ws_bytes, need);
    if (!aligned(ws, kWsAlign)) return fail(PTQ1_ERR_ALIGN, "%s: ws is not 256-byte aligned", fn);
    return PTQ1_OK;
}

#define PTQ1_TRY(expr)                         \
    do {                                       \
        const ptq1_status _s = (expr);         \
        if (_s != PTQ1_OK) return _s;          \
    } while (0)

int64_t nseg_of(int64_t k) { return (k + ptq1::kHadamard - 1) / ptq1::kHadamard; }

// ---- workspace layouts -------------------------------------------------------
// lookup-table decode: split-K partials [slice][matrix][row]
size_t lut_ws(int64_t n, int nmat, int64_t k)
{
    return round_up(ptq1::lut_part_floats(n, nmat, k) * sizeof(float), kWsAlign);
}

// GEMM: bf16 activation fragments, then the partial tiles of tiles that
// several workgroups share (two per workgroup at most)
struct GemmWs {
    size_t frag = 0, part = 0, total = 0;  // byte offsets
};

GemmWs gemm_layout(const ptq1::GemmPlan &p, int64_t k)
{
    GemmWs L;
    L.frag = 0;
    L.part = round_up(ptq1::gemm_frag_elems(p, k) * 2, kWsAlign);
    L.total = L.part + round_up(ptq1::gemm_part_floats(p) * sizeof(float), kWsAlign);
    return L;
}

struct FfnWs {
    size_t part = 0, hr = 0, g = 0, u = 0, xb = 0, total = 0;  // byte offsets (hr: h at m = 1)
    ptq1::GemmPlan gu, dn;                                      // m >= 2: gate+up and down GEMMs
};

// rd_only: the PQ2_0 block (register-decode GEMM plans at every m)
FfnWs ffn_layout(int64_t m, int64_t d, int64_t f, bool rd_only = false)
{
    FfnWs L;
    size_t off = 0;
    if (m == 1) {
        const size_t part_a = lut_ws(f, 2, d), part_b = lut_ws(d, 1, f);
        L.part = off;
        off += part_a > part_b ? part_a : part_b;
        L.hr = off; off += round_up(static_cast<size_t>(f) * 4, kWsAlign);
    } else {
        L.gu = ptq1::gemm_plan(m, 2 * f, d, rd_only);
        L.dn = ptq1::gemm_plan(m, d, f, rd_only);
        const size_t fa = ptq1::gemm_frag_elems(L.gu, d), fb = ptq1::gemm_frag_elems(L.dn, f);
        const size_t pa = ptq1::gemm_part_floats(L.gu), pb = ptq1::gemm_part_floats(L.dn);
        L.xb = off; off += round_up((fa > fb ? fa : fb) * 2, kWsAlign);
        L.g = off; off += round_up(static_cast<size_t>(m) * f * 4, kWsAlign);
        L.u = off; off += round_up(static_cast<size_t>(m) * f * 4, kWsAlign);
        L.part = off; off += round_up((pa > pb ? pa : pb) * sizeof(float), kWsAlign);
    }
    L.total = off;
    return L;
}

// ---- profiling hook ----------------------------------------------------------
// Armed kernel families record caller events around their next launches.
enum ProfKind { kProfLut2 = 0, kProfLut1 = 1, kProfGemm = 2, kProfPq2 = 3, kProfPeel = 4, kProfKinds = 5 };
const char *const kProfNames[kProfKinds] = {"lut_matvec_2", "lut_matvec_1", "gemm", "pq2_matvec", "peel_matvec"};

struct ProfArm {
    hipEvent_t *start = nullptr, *stop = nullptr;
    int32_t count = 0, next = 0;
};

std::mutex g_prof_mu;
ProfArm g_prof[kProfKinds];
std::atomic<bool> g_prof_any{false};

int prof_kind(const char *name)
{
    for (int i = 0; i < kProfKinds; ++i)
        if (std::strcmp(name, kProfNames[i]) == 0) return i;
    return -1;
}

// Runs `launch` with the family's next pair of events attached to its
// kernel dispatch, if the family is armed.
template <class F>
hipError_t profiled(int kind, hipStream_t s, F launch)
{
    (void)s;
    if (!g_prof_any.load(std::memory_order_relaxed)) return launch();
    ptq1::ProfEvents ev;
    {
        std::lock_guard<std::mutex> lk(g_prof_mu);
        ProfArm &p = g_prof[kind];
        if (p.next < p.count) {
            ev.start = p.start[p.next];
            ev.stop = p.stop[p.next];
            ++p.next;
        }
    }
    ptq1::prof_events() = ev;
    const hipError_t e = launch();
    ptq1::prof_events() = ptq1::ProfEvents{};
    return e;
}

}  // namespace

namespace ptq1 {
ProfEvents &prof_events()
{
    thread_local ProfEvents ev;
    return ev;
}

hipError_t allow_dynamic_lds(const void *kernel, int bytes, std::atomic<uint64_t> &done_mask)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = dev >= 0 && dev < 64 ? uint64_t{1} << dev : 0;
    if (bit != 0 && (done_mask.load(std::memory_order_acquire) & bit)) return hipSuccess;
    e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess && bit != 0) done_mask.fetch_or(bit, std::memory_order_release);
    return e;
}
}  // namespace ptq1

extern "C" {

ptq1_status ptq1_profile_arm(const char *kernel, hipEvent_t *start, hipEvent_t *stop, int32_t count)
{
    if (kernel == nullptr) return fail(PTQ1_ERR_NULL, "kernel is NULL");
    const int kind = prof_kind(kernel);
    if (kind < 0) return fail(PTQ1_ERR_UNSUPPORTED, "no kernel family named '%s'", kernel);
    if (count < 0) return fail(PTQ1_ERR_SHAPE, "count = %d is negative", count);
    if (count > 0 && (start == nullptr || stop == nullptr)) return fail(PTQ1_ERR_NULL, "start or stop is NULL");
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof[kind] = ProfArm{count > 0 ? start : nullptr, count > 0 ? stop : nullptr, count, 0};
    bool any = false;
    for (const ProfArm &p : g_prof) any = any || p.count > 0;
    g_prof_any.store(any, std::memory_order_relaxed);
    return ok();
}

int32_t ptq1_profile_count(const char *kernel)
{
    const int kind = kernel ? prof_kind(kernel) : -1;
    if (kind < 0) return -1;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    return g_prof[kind].next;
}

const char *ptq1_status_string(ptq1_status s)
{
    switch (s) {
        case PTQ1_OK: return "PTQ1_OK";
        case PTQ1_ERR_NULL: return "PTQ1_ERR_NULL";
        case PTQ1_ERR_SHAPE: return "PTQ1_ERR_SHAPE";
        case PTQ1_ERR_ALIGN: return "PTQ1_ERR_ALIGN";
        case PTQ1_ERR_OVERFLOW: return "PTQ1_ERR_OVERFLOW";
        case PTQ1_ERR_UNSUPPORTED: return "PTQ1_ERR_UNSUPPORTED";
        case PTQ1_ERR_WORKSPACE: return "PTQ1_ERR_WORKSPACE";
        case PTQ1_ERR_ALIAS: return "PTQ1_ERR_ALIAS";
        case PTQ1_ERR_HIP: return "PTQ1_ERR_HIP";
    }
    return "PTQ1_ERR_UNKNOWN";
}

const char *ptq1_last_error(void) { return g_last_error.c_str(); }

ptq1_status ptq1_geometry(int32_t *out, int32_t n)
{
    if (out == nullptr) return fail(PTQ1_ERR_NULL, "out is NULL");
    if (n < 0 || n > 6) return fail(PTQ1_ERR_SHAPE, "n = %d outside [0, 6]", n);
    const int32_t g[6] = {ptq1::kBlockWeights, ptq1::kTritBytes, ptq1::kBlockBytes,
                          ptq1::kHadamard,     ptq1::kTileRows,  ptq1::kTileBlocks};
    for (int32_t i = 0; i < n; ++i) out[i] = g[i];
    return ok();
}

int64_t ptq1_packed_bytes(int64_t n, int64_t k) { return packed_bytes(n, k); }

int64_t ptq1_tiled_bytes(int64_t n, int64_t k) { return packed_bytes(n, k) < 0 ? -1 : tiled_bytes(n, k); }

ptq1_status ptq1_tile(const uint8_t *blocks, int64_t n, int64_t k, uint8_t *tiled, hipStream_t stream)
{
    int64_t pb, tb;
    PTQ1_TRY(check_matrix(blocks, "blocks", n, k, false, &pb));
    PTQ1_TRY(check_matrix(tiled, "tiled", n, k, false, &tb, true));
    if (tb == 0) return ok();
    if (overlaps(tiled, tb, blocks, pb)) return fail(PTQ1_ERR_ALIAS, "tiled overlaps blocks");
    return hip_status(ptq1::launch_tile(blocks, n, k, tiled, stream), "ptq1_tile");
}

ptq1_status ptq1_pack(const int8_t *trits, const uint16_t *scales_f16, int64_t n, int64_t k,
                      uint8_t *blocks, hipStream_t stream)
{
    int64_t bytes;
    PTQ1_TRY(check_matrix(blocks, "blocks", n, k, false, &bytes));
    if (bytes == 0) return ok();
    int64_t nt;
    if (!mul_ok(n, k, &nt)) return fail(PTQ1_ERR_OVERFLOW, "trits: n * k overflows");
    if (trits == nullptr) return fail(PTQ1_ERR_NULL, "trits is NULL");
    if (scales_f16 == nullptr) return fail(PTQ1_ERR_NULL, "scales_f16 is NULL");
    if (!aligned(scales_f16, 2)) return fail(PTQ1_ERR_ALIGN, "scales_f16 is not 2-byte aligned");
    const int64_t ns = n * (k / ptq1::kBlockWeights);
    if (overlaps(blocks, bytes, trits, nt) || overlaps(blocks, bytes, scales_f16, 2 * ns))
        return fail(PTQ1_ERR_ALIAS, "blocks overlaps an input");
    return hip_status(ptq1::launch_pack(trits, scales_f16, n, k, blocks, stream), "ptq1_pack");
}

ptq1_status ptq1_dequant(const uint8_t *blocks, int64_t n, int64_t k, float *w, hipStream_t stream)
{
    int64_t bytes, wb, nk;
    PTQ1_TRY(check_matrix(blocks, "blocks", n, k, false, &bytes));
    if (!mul_ok(n, k, &nk)) return fail(PTQ1_ERR_OVERFLOW, "w: n * k overflows");
    PTQ1_TRY(check_floats(w, "w", nk, &wb));
    if (nk == 0) return ok();
    if (overlaps(w, wb, blocks, bytes)) return fail(PTQ1_ERR_ALIAS, "w overlaps blocks");
    return hip_status(ptq1::launch_dequant(blocks, n, k, w, stream), "ptq1_dequant");
}

ptq1_status hadamard_rotate(const float *x, float *y, int64_t m, int64_t k, const float *signs1024,
                            hipStream_t stream)
{
    if (m < 0 || k < 0) return fail(PTQ1_ERR_SHAPE, "m or k is negative");
    if (k % ptq1::kHadamard != 0)
        return fail(PTQ1_ERR_SHAPE, "k = %lld is not a multiple of %d", (long long)k, ptq1::kHadamard);
    int64_t mk, xb, yb;
    if (!mul_ok(m, k, &mk)) return fail(PTQ1_ERR_OVERFLOW, "m * k overflows");
    PTQ1_TRY(check_floats(x, "x", mk, &xb));
    PTQ1_TRY(check_floats(y, "y", mk, &yb));
    if (mk == 0) return ok();
    PTQ1_TRY(check_signs(signs1024, true));
    if (x != y && overlaps(x, xb, y, yb)) return fail(PTQ1_ERR_ALIAS, "y partially overlaps x");
    if (overlaps(y, yb, signs1024, 4 * ptq1::kHadamard)) return fail(PTQ1_ERR_ALIAS, "y overlaps signs1024");
    if (mk / ptq1::kHadamard > kMaxGridX) return fail(PTQ1_ERR_UNSUPPORTED, "more than 2^31-1 chunks");
    return hip_status(ptq1::launch_rotate(x, y, m, k, signs1024, stream), "hadamard_rotate");
}

ptq1_status hadamard_unrotate_rows(const float *table, int64_t n_table, int64_t d,
                                   const int32_t *ids, int64_t n_rows, const float *signs1024,
                                   float *out, hipStream_t stream)
{
    if (n_table < 0 || d < 0 || n_rows < 0) return fail(PTQ1_ERR_SHAPE, "negative size");
    if (d % ptq1::kHadamard != 0)
        return fail(PTQ1_ERR_SHAPE, "d = %lld is not a multiple of %d", (long long)d, ptq1::kHadamard);
    if (ids == nullptr && n_rows > n_table)
        return fail(PTQ1_ERR_SHAPE, "n_rows = %lld > n_table = %lld without ids", (long long)n_rows,
                    (long long)n_table);
    int64_t tn, on, tb, ob;
    if (!mul_ok(n_table, d, &tn)) return fail(PTQ1_ERR_OVERFLOW, "n_table * d overflows");
    if (!mul_ok(n_rows, d, &on)) return fail(PTQ1_ERR_OVERFLOW, "n_rows * d overflows");
    PTQ1_TRY(check_floats(out, "out", on, &ob));
    if (on == 0) return ok();
    PTQ1_TRY(check_floats(table, "table", tn, &tb));
    if (tn == 0 && ids == nullptr) return fail(PTQ1_ERR_SHAPE, "empty table");
    PTQ1_TRY(check_signs(signs1024, true));
    if (ids != nullptr && !aligned(ids, 4)) return fail(PTQ1_ERR_ALIGN, "ids is not 4-byte aligned");
    if (overlaps(out, ob, table, tb)) return fail(PTQ1_ERR_ALIAS, "out overlaps table");
    if (ids != nullptr && overlaps(out, ob, ids, 4 * n_rows)) return fail(PTQ1_ERR_ALIAS, "out overlaps ids");
    if (on / ptq1::kHadamard > kMaxGridX) return fail(PTQ1_ERR_UNSUPPORTED, "more than 2^31-1 chunks");
    return hip_status(ptq1::launch_unrotate_rows(table, n_table, d, ids, n_rows, signs1024, out, stream),
                      "hadamard_unrotate_rows");
}

size_t ptq1_matvec_workspace_bytes(int64_t n, int64_t k)
{
    if (packed_bytes(n, k) < 0) return 0;
    return lut_ws(n, 1, k);
}

namespace {

ptq1_status check_matvec(const uint8_t *blocks, int64_t n, int64_t k, const float *x,
                         const float *signs1024, const float *residual, float *y, void *ws,
                         size_t ws_bytes, const char *fn, bool tiled, bool *empty)
{
    int64_t wb, xb, yb;
    *empty = false;
    PTQ1_TRY(check_matrix(blocks, tiled ? "tiled" : "blocks", n, k, signs1024 != nullptr, &wb, tiled));
    PTQ1_TRY(check_floats(y, "y", n, &yb));
    if (n == 0) {
        *empty = true;
        return ok();
    }
    PTQ1_TRY(check_floats(x, "x", k, &xb));
    PTQ1_TRY(check_signs(signs1024, false));
    if (residual != nullptr) {
        int64_t rb;
        PTQ1_TRY(check_floats(residual, "residual", n, &rb));
        if (residual != y && overlaps(residual, rb, y, yb))
            return fail(PTQ1_ERR_ALIAS, "y partially overlaps residual");
    }
    const size_t need = ptq1_matvec_workspace_bytes(n, k);
    PTQ1_TRY(check_ws(ws, ws_bytes, need, fn));
    if (overlaps(y, yb, x, xb)) return fail(PTQ1_ERR_ALIAS, "y overlaps x");
    if (overlaps(y, yb, blocks, wb)) return fail(PTQ1_ERR_ALIAS, "y overlaps the weights");
    if (overlaps(ws, (int64_t)need, y, yb) || overlaps(ws, (int64_t)need, x, xb) ||
        overlaps(ws, (int64_t)need, blocks, wb))
        return fail(PTQ1_ERR_ALIAS, "ws overlaps an argument");
    if (nseg_of(k) * 4 > kMaxGridY) return fail(PTQ1_ERR_UNSUPPORTED, "k = %lld too large", (long long)k);
    if (n > kMaxLutRows) return fail(PTQ1_ERR_UNSUPPORTED, "n = %lld > %lld rows", (long long)n, (long long)kMaxLutRows);
    if (tiled && wb > kMaxLutMatrixBytes) return fail(PTQ1_ERR_UNSUPPORTED, "tiled matrix above 2 GiB");
    return PTQ1_OK;
}

}  // namespace

ptq1_status ptq1_matvec(const uint8_t *tiled, int64_t n, int64_t k, const float *x,
                        const float *signs1024, const float *residual, float *y, void *ws,
                        size_t ws_bytes, hipStream_t stream)
{
    bool empty;
    PTQ1_TRY(check_matvec(tiled, n, k, x, signs1024, residual, y, ws, ws_bytes, "ptq1_matvec", true, &empty));
    if (empty) return ok();
    float *part = static_cast<float *>(ws);
    hipError_t e = profiled(kProfLut1, stream, [&] {
        return ptq1::launch_matvec_lut(tiled, nullptr, 1, n, k, x, signs1024, nullptr, part, stream);
    });
    if (e == hipSuccess) e = ptq1::launch_lut_sum_rows(part, n, k, residual, y, stream);
    return hip_status(e, "ptq1_matvec");
}

ptq1_status ptq1_matvec_float_peel(const uint8_t *tiled, int64_t n, int64_t k, const float *x,
                                   const float *signs1024, const float *residual, float *y, void *ws,
                                   size_t ws_bytes, hipStream_t stream)
{
    bool empty;
    PTQ1_TRY(check_matvec(tiled, n, k, x, signs1024, residual, y, ws, ws_bytes, "ptq1_matvec_float_peel", true,
                          &empty));
    if (empty) return ok();
    float *part = static_cast<float *>(ws);
    hipError_t e = profiled(kProfPeel, stream, [&] {
        return ptq1::launch_matvec_peel(tiled, nullptr, 1, n, k, x, signs1024, nullptr, part, stream);
    });
    if (e == hipSuccess) e = ptq1::launch_lut_sum_rows(part, n, k, residual, y, stream);
    return hip_status(e, "ptq1_matvec_float_peel");
}

size_t ptq1_gate_up_workspace_bytes(int64_t f, int64_t d)
{
    if (packed_bytes(f, d) < 0 || f > INT64_MAX / 2) return 0;
    return lut_ws(f, 2, d);
}

ptq1_status ptq1_gate_up(const uint8_t *w_gate, const uint8_t *w_up, int64_t f, int64_t d,
                         const float *x, const float *signs1024, float *g, float *u, void *ws,
                         size_t ws_bytes, hipStream_t stream)
{
    int64_t wgb, wub, xb, gb, ub;
    PTQ1_TRY(check_matrix(w_gate, "w_gate", f, d, signs1024 != nullptr, &wgb, true));
    PTQ1_TRY(check_matrix(w_up, "w_up", f, d, signs1024 != nullptr, &wub, true));
    PTQ1_TRY(check_floats(g, "g", f, &gb));
    PTQ1_TRY(check_floats(u, "u", f, &ub));
    if (f == 0) return ok();
    PTQ1_TRY(check_floats(x, "x", d, &xb));
    PTQ1_TRY(check_signs(signs1024, false));
    const size_t need = lut_ws(f, 2, d);
    PTQ1_TRY(check_ws(ws, ws_bytes, need, "ptq1_gate_up"));
    if (overlaps(g, gb, u, ub)) return fail(PTQ1_ERR_ALIAS, "g overlaps u");
    if (overlaps(g, gb, x, xb) || overlaps(u, ub, x, xb)) return fail(PTQ1_ERR_ALIAS, "g or u overlaps x");
    if (overlaps(ws, (int64_t)need, g, gb) || overlaps(ws, (int64_t)need, u, ub) ||
        overlaps(ws, (int64_t)need, x, xb))
        return fail(PTQ1_ERR_ALIAS, "ws overlaps an argument");
    if (nseg_of(d) * 4 > kMaxGridY) return fail(PTQ1_ERR_UNSUPPORTED, "d = %lld too large", (long long)d);
    if (f > kMaxLutRows) return fail(PTQ1_ERR_UNSUPPORTED, "f = %lld > %lld rows", (long long)f, (long long)kMaxLutRows);
    if (wgb > kMaxLutMatrixBytes) return fail(PTQ1_ERR_UNSUPPORTED, "tiled matrices above 2 GiB");
    float *part = static_cast<float *>(ws);
    hipError_t e = profiled(kProfLut2, stream, [&] {
        return ptq1::launch_matvec_lut(w_gate, w_up, 2, f, d, x, signs1024, nullptr, part, stream);
    });
    if (e == hipSuccess)
        e = ptq1::launch_lut_gate_up_sum(part, f, d, nullptr, 0, 0.0f, g, u, nullptr, stream);
    return hip_status(e, "ptq1_gate_up");
}

ptq1_status ptq1_swiglu(const float *g, const float *u, float *h, int64_t len, hipStream_t stream)
{
    int64_t gb, ub, hb;
    PTQ1_TRY(check_floats(g, "g", len, &gb));
    PTQ1_TRY(check_floats(u, "u", len, &ub));
    PTQ1_TRY(check_floats(h, "h", len, &hb));
    if (len == 0) return ok();
    if ((h != g && overlaps(h, hb, g, gb)) || (h != u && overlaps(h, hb, u, ub)))
        return fail(PTQ1_ERR_ALIAS, "h partially overlaps g or u");
    return hip_status(ptq1::launch_swiglu(g, u, h, len, stream), "ptq1_swiglu");
}

size_t ptq1_gemm_workspace_bytes(int64_t m, int64_t n, int64_t k)
{
    if (packed_bytes(n, k) < 0 || m < 0 || m > kMaxGemmM) return 0;
    if (m == 0) return 0;
    return gemm_layout(ptq1::gemm_plan(m, n, k), k).total;
}

ptq1_status ptq1_gemm(const uint8_t *tiled, int64_t n, int64_t k, const float *x, int64_t m,
                      const float *signs1024, float *y, void *ws, size_t ws_bytes, hipStream_t stream)
{
    int64_t wb, mk, mn, xb, yb;
    PTQ1_TRY(check_matrix(tiled, "tiled", n, k, signs1024 != nullptr, &wb, true));
    if (m < 0) return fail(PTQ1_ERR_SHAPE, "m = %lld is negative", (long long)m);
    if (m > kMaxGemmM) return fail(PTQ1_ERR_UNSUPPORTED, "m = %lld > %lld", (long long)m, (long long)kMaxGemmM);
    if (!mul_ok(m, k, &mk) || !mul_ok(m, n, &mn)) return fail(PTQ1_ERR_OVERFLOW, "m * k or m * n overflows");
    PTQ1_TRY(check_floats(y, "y", mn, &yb));
    if (mn == 0) return ok();
    PTQ1_TRY(check_floats(x, "x", mk, &xb));
    PTQ1_TRY(check_signs(signs1024, false));
    const ptq1::GemmPlan plan = ptq1::gemm_plan(m, n, k);
    const GemmWs L = gemm_layout(plan, k);
    const size_t need = L.total;
    PTQ1_TRY(check_ws(ws, ws_bytes, need, "ptq1_gemm"));
    if (overlaps(y, yb, x, xb)) return fail(PTQ1_ERR_ALIAS, "y overlaps x");
    if (overlaps(y, yb, tiled, wb)) return fail(PTQ1_ERR_ALIAS, "y overlaps tiled");
    if (overlaps(ws, (int64_t)need, y, yb) || overlaps(ws, (int64_t)need, x, xb) ||
        overlaps(ws, (int64_t)need, tiled, wb))
        return fail(PTQ1_ERR_ALIAS, "ws overlaps an argument");
    char *w = static_cast<char *>(ws);
    uint16_t *xf = reinterpret_cast<uint16_t *>(w + L.frag);
    float *part = reinterpret_cast<float *>(w + L.part);
    hipError_t e = ptq1::launch_prep_frag(x, nullptr, nullptr, m, k, signs1024, 0.0f, nullptr, xf, stream);
    if (e == hipSuccess)
        e = profiled(kProfGemm, stream, [&] {
            return ptq1::launch_gemm(plan, xf, m, tiled, n, nullptr, 0, y, nullptr, nullptr, part, stream);
        });
    return hip_status(e, "ptq1_gemm");
}

size_t ptq1_ffn_workspace_bytes(int64_t m, int64_t d, int64_t f)
{
    if (m < 0 || m > kMaxGemmM || packed_bytes(f, d) < 0 || packed_bytes(d, f) < 0 || f > INT64_MAX / 2)
        return 0;
    if (m == 0) return 0;
    return ffn_layout(m, d, f).total;
}

static ptq1_status ffn_block_impl(const float *x, float *x_out, int64_t m, int64_t d, int64_t f,
                                  const uint8_t *w_gate, const uint8_t *w_up, const uint8_t *w_down,
                                  const float *signs1024, float rms_eps, const float *rms_gain, void *ws,
                                  size_t ws_bytes, hipStream_t stream, bool scratch)
{
    int64_t wgb, wub, wdb, md, xb, ob;
    if (m < 0) return fail(PTQ1_ERR_SHAPE, "m = %lld is negative", (long long)m);
    if (m > kMaxGemmM) return fail(PTQ1_ERR_UNSUPPORTED, "m = %lld > %lld", (long long)m, (long long)kMaxGemmM);
    PTQ1_TRY(check_matrix(w_gate, "w_gate", f, d, true, &wgb, true));
    PTQ1_TRY(check_matrix(w_up, "w_up", f, d, true, &wub, true));
    PTQ1_TRY(check_matrix(w_down, "w_down", d, f, true, &wdb, true));
    if (!mul_ok(m, d, &md)) return fail(PTQ1_ERR_OVERFLOW, "m * d overflows");
    PTQ1_TRY(check_floats(x_out, "x_out", md, &ob));
    if (md == 0) return ok();
    PTQ1_TRY(check_floats(x, "x", md, &xb));
    PTQ1_TRY(check_signs(signs1024, true));
    int64_t gb = 0;
    if (rms_gain != nullptr) {
        PTQ1_TRY(check_floats(rms_gain, "rms_gain", d, &gb));
        if (overlaps(x_out, ob, rms_gain, gb)) return fail(PTQ1_ERR_ALIAS, "x_out overlaps rms_gain");
    }
    if (x_out != x && overlaps(x_out, ob, x, xb)) return fail(PTQ1_ERR_ALIAS, "x_out partially overlaps x");
    if (overlaps(x_out, ob, w_gate, wgb) || overlaps(x_out, ob, w_up, wub) || overlaps(x_out, ob, w_down, wdb))
        return fail(PTQ1_ERR_ALIAS, "x_out overlaps a weight matrix");
    if (f == 0) return fail(PTQ1_ERR_SHAPE, "f = 0");
    const FfnWs L = ffn_layout(m, d, f);
    if (scratch) {
        if (L.total > ptq1::kScratchBytes)
            return fail(PTQ1_ERR_UNSUPPORTED,
                        "ptq1_ffn_block_noalloc: m = %lld, d = %lld, f = %lld needs %zu bytes of scratch, more than "
                        "the library's %zu (use ptq1_ffn_block with a workspace)",
                        (long long)m, (long long)d, (long long)f, L.total, ptq1::kScratchBytes);
        const hipError_t es = ptq1::scratch_device_ptr(&ws);
        if (es != hipSuccess) return hip_status(es, "ptq1_ffn_block_noalloc: scratch address");
        ws_bytes = ptq1::kScratchBytes;
    }
    PTQ1_TRY(check_ws(ws, ws_bytes, L.total, scratch ? "ptq1_ffn_block_noalloc" : "ptq1_ffn_block"));
    if (overlaps(ws, (int64_t)L.total, x, xb) || overlaps(ws, (int64_t)L.total, x_out, ob))
        return fail(PTQ1_ERR_ALIAS, "ws overlaps x or x_out");
    if (rms_gain != nullptr && overlaps(ws, (int64_t)L.total, rms_gain, gb))
        return fail(PTQ1_ERR_ALIAS, "ws overlaps rms_gain");
    if (nseg_of(f) * 4 > kMaxGridY || nseg_of(d) * 4 > kMaxGridY)
        return fail(PTQ1_ERR_UNSUPPORTED, "d or f too large");
    if (m == 1 && (f > kMaxLutRows || d > kMaxLutRows))
        return fail(PTQ1_ERR_UNSUPPORTED, "d or f > %lld rows", (long long)kMaxLutRows);
    if (m == 1 && (wgb > kMaxLutMatrixBytes || wdb > kMaxLutMatrixBytes))
        return fail(PTQ1_ERR_UNSUPPORTED, "tiled matrices above 2 GiB");
    char *w = static_cast<char *>(ws);
    hipError_t e;
    if (m == 1) {
        // gate/up partials -> RMS scale and SwiGLU -> down partials over R h -> + x
        float *part = reinterpret_cast<float *>(w + L.part);
        float *h = reinterpret_cast<float *>(w + L.hr);
        e = profiled(kProfLut2, stream, [&] {
            return ptq1::launch_matvec_lut(w_gate, w_up, 2, f, d, x, signs1024, rms_gain, part, stream);
        });
        if (e == hipSuccess)
            e = ptq1::launch_lut_gate_up_sum(part, f, d, rms_eps > 0.0f ? x : nullptr, d, rms_eps, nullptr, nullptr,
                                             h, stream);
        if (e == hipSuccess)
            e = profiled(kProfLut1, stream, [&] {
                return ptq1::launch_matvec_lut(w_down, nullptr, 1, d, f, h, signs1024, nullptr, part, stream);
            });
        if (e == hipSuccess) e = ptq1::launch_lut_sum_rows(part, d, f, x, x_out, stream);
    } else {
        uint16_t *xf = reinterpret_cast<uint16_t *>(w + L.xb);
        float *g = reinterpret_cast<float *>(w + L.g);
        float *u = reinterpret_cast<float *>(w + L.u);
        float *part = reinterpret_cast<float *>(w + L.part);
        // the gate+up GEMM's fix-up is taken over by the prep of silu(g) u
        // when its shared tiles are narrow enough (one kernel fewer)
        const bool fold = ptq1::gemm_fold_ok(L.gu);
        e = ptq1::launch_prep_frag(x, nullptr, nullptr, m, d, signs1024, rms_eps, rms_gain, xf, stream);
        if (e == hipSuccess)
            e = profiled(kProfGemm, stream, [&] {
                return ptq1::launch_gemm(L.gu, xf, m, w_gate, f, w_up, f, g, u, nullptr, part, stream, !fold);
            });
        if (e == hipSuccess)
            e = ptq1::launch_prep_frag(nullptr, g, u, m, f, signs1024, 0.0f, nullptr, xf, stream,
                                       fold ? ptq1::gemm_sk_view(L.gu, part) : ptq1::SkView{});
        if (e == hipSuccess)
            e = profiled(kProfGemm, stream, [&] {
                return ptq1::launch_gemm(L.dn, xf, m, w_down, d, nullptr, 0, x_out, nullptr, x, part, stream);
            });
    }
    return hip_status(e, scratch ? "ptq1_ffn_block_noalloc" : "ptq1_ffn_block");
}

ptq1_status ptq1_ffn_block(const float *x, float *x_out, int64_t m, int64_t d, int64_t f,
                           const uint8_t *w_gate, const uint8_t *w_up, const uint8_t *w_down,
                           const float *signs1024, float rms_eps, const float *rms_gain, void *ws,
                           size_t ws_bytes, hipStream_t stream)
{
    return ffn_block_impl(x, x_out, m, d, f, w_gate, w_up, w_down, signs1024, rms_eps, rms_gain, ws, ws_bytes, stream,
                          false);
}

ptq1_status ptq1_ffn_block_noalloc(const float *x, float *x_out, int64_t m, int64_t d, int64_t f,
                                   const uint8_t *w_gate, const uint8_t *w_up, const uint8_t *w_down,
                                   const float *signs1024, float rms_eps, const float *rms_gain, hipStream_t stream)
{
    return ffn_block_impl(x, x_out, m, d, f, w_gate, w_up, w_down, signs1024, rms_eps, rms_gain, nullptr, 0, stream,
                          true);
}

namespace {

ptq1_status ffn_offsets(int64_t m, int64_t d, int64_t f, bool rd_only, int64_t *offsets, const char *fn)
{
    if (offsets == nullptr) return fail(PTQ1_ERR_NULL, "%s: offsets is NULL", fn);
    if (m < 1 || d < 0 || f < 1) return fail(PTQ1_ERR_SHAPE, "%s: m = %lld, d = %lld, f = %lld", fn, (long long)m,
                                             (long long)d, (long long)f);
    if (m > kMaxGemmM) return fail(PTQ1_ERR_UNSUPPORTED, "%s: m = %lld > %lld", fn, (long long)m, (long long)kMaxGemmM);
    if (d % ptq1::kHadamard != 0 || f % ptq1::kHadamard != 0)
        return fail(PTQ1_ERR_SHAPE, "%s: d and f must be multiples of %d", fn, ptq1::kHadamard);
    const FfnWs L = ffn_layout(m, d, f, rd_only);
    offsets[0] = m >= 2 ? static_cast<int64_t>(L.g) : -1;
    offsets[1] = m >= 2 ? static_cast<int64_t>(L.u) : -1;
    offsets[2] = m == 1 ? static_cast<int64_t>(L.hr) : -1;
    return ok();
}

}  // namespace

ptq1_status ptq1_ffn_workspace_offsets(int64_t m, int64_t d, int64_t f, int64_t *offsets)
{
    return ffn_offsets(m, d, f, false, offsets, "ptq1_ffn_workspace_offsets");
}

ptq1_status pq2_ffn_workspace_offsets(int64_t m, int64_t d, int64_t f, int64_t *offsets)
{
    return ffn_offsets(m, d, f, true, offsets, "pq2_ffn_workspace_offsets");
}

// ---- PQ2_0 ------------------------------------------------------------------

int64_t pq2_packed_bytes(int64_t n, int64_t k) { return pq2_packed(n, k); }

int64_t pq2_tiled_bytes(int64_t n, int64_t k) { return pq2_tiled(n, k); }

ptq1_status pq2_pack(const int8_t *trits, const uint16_t *scales_f16, int64_t n, int64_t k, uint8_t *blocks,
                     hipStream_t stream)
{
    int64_t bytes;
    PTQ1_TRY(check_pq2(blocks, "blocks", n, k, false, &bytes, false));
    if (bytes == 0) return ok();
    int64_t nt;
    if (!mul_ok(n, k, &nt)) return fail(PTQ1_ERR_OVERFLOW, "trits: n * k overflows");
    if (trits == nullptr) return fail(PTQ1_ERR_NULL, "trits is NULL");
    if (scales_f16 == nullptr) return fail(PTQ1_ERR_NULL, "scales_f16 is NULL");
    if (!aligned(scales_f16, 2)) return fail(PTQ1_ERR_ALIGN, "scales_f16 is not 2-byte aligned");
    const int64_t ns = n * (k / ptq1::kBlockWeights);
    if (overlaps(blocks, bytes, trits, nt) || overlaps(blocks, bytes, scales_f16, 2 * ns))
        return fail(PTQ1_ERR_ALIAS, "blocks overlaps an input");
    return hip_status(ptq1::launch_pq2_pack(trits, scales_f16, n, k, blocks, stream), "pq2_pack");
}

ptq1_status pq2_dequant(const uint8_t *blocks, int64_t n, int64_t k, float *w, hipStream_t stream)
{
    int64_t bytes, wb, nk;
    PTQ1_TRY(check_pq2(blocks, "blocks", n, k, false, &bytes, false));
    if (!mul_ok(n, k, &nk)) return fail(PTQ1_ERR_OVERFLOW, "w: n * k overflows");
    PTQ1_TRY(check_floats(w, "w", nk, &wb));
    if (nk == 0) return ok();
    if (overlaps(w, wb, blocks, bytes)) return fail(PTQ1_ERR_ALIAS, "w overlaps blocks");
    return hip_status(ptq1::launch_pq2_dequant(blocks, n, k, w, stream), "pq2_dequant");
}

ptq1_status pq2_tile(const uint8_t *blocks, int64_t n, int64_t k, uint8_t *tiled, hipStream_t stream)
{
    int64_t pb, tb;
    PTQ1_TRY(check_pq2(blocks, "blocks", n, k, false, &pb, false));
    PTQ1_TRY(check_pq2(tiled, "tiled", n, k, false, &tb, true));
    if (tb == 0) return ok();
    if (overlaps(tiled, tb, blocks, pb)) return fail(PTQ1_ERR_ALIAS, "tiled overlaps blocks");
    return hip_status(ptq1::launch_pq2_tile(blocks, n, k, tiled, stream), "pq2_tile");
}

size_t pq2_matvec_workspace_bytes(int64_t n, int64_t k)
{
    if (pq2_packed(n, k) < 0) return 0;
    return lut_ws(n, 1, k);
}

ptq1_status pq2_matvec(const uint8_t *tiled, int64_t n, int64_t k, const float *x, const float *signs1024,
                       const float *residual, float *y, void *ws, size_t ws_bytes, hipStream_t stream)
{
    int64_t wb, xb, yb;
    PTQ1_TRY(check_pq2(tiled, "tiled", n, k, signs1024 != nullptr, &wb, true));
    PTQ1_TRY(check_floats(y, "y", n, &yb));
    if (n == 0) return ok();
    PTQ1_TRY(check_floats(x, "x", k, &xb));
    PTQ1_TRY(check_signs(signs1024, false));
    if (residual != nullptr) {
        int64_t rb;
        PTQ1_TRY(check_floats(residual, "residual", n, &rb));
        if (residual != y && overlaps(residual, rb, y, yb))
            return fail(PTQ1_ERR_ALIAS, "y partially overlaps residual");
    }
    const size_t need = pq2_matvec_workspace_bytes(n, k);
    PTQ1_TRY(check_ws(ws, ws_bytes, need, "pq2_matvec"));
    if (overlaps(y, yb, x, xb)) return fail(PTQ1_ERR_ALIAS, "y overlaps x");
    if (overlaps(y, yb, tiled, wb)) return fail(PTQ1_ERR_ALIAS, "y overlaps the weights");
    if (overlaps(ws, (int64_t)need, y, yb) || overlaps(ws, (int64_t)need, x, xb) ||
        overlaps(ws, (int64_t)need, tiled, wb))
        return fail(PTQ1_ERR_ALIAS, "ws overlaps an argument");
    if (nseg_of(k) * 4 > kMaxGridY) return fail(PTQ1_ERR_UNSUPPORTED, "k = %lld too large", (long long)k);
    if (n > kMaxLutRows) return fail(PTQ1_ERR_UNSUPPORTED, "n = %lld > %lld rows", (long long)n, (long long)kMaxLutRows);
    if (wb > kMaxLutMatrixBytes) return fail(PTQ1_ERR_UNSUPPORTED, "tiled matrix above 2 GiB");
    float *part = static_cast<float *>(ws);
    hipError_t e = profiled(kProfPq2, stream, [&] {
        return ptq1::launch_pq2_matvec(tiled, nullptr, 1, n, k, x, signs1024, nullptr, part, stream);
    });
    if (e == hipSuccess) e = ptq1::launch_lut_sum_rows(part, n, k, residual, y, stream);
    return hip_status(e, "pq2_matvec");
}

size_t pq2_gemm_workspace_bytes(int64_t m, int64_t n, int64_t k)
{
    if (pq2_packed(n, k) < 0 || m < 0 || m > kMaxGemmM) return 0;
    if (m == 0) return 0;
    return gemm_layout(ptq1::gemm_plan(m, n, k, true), k).total;
}

ptq1_status pq2_gemm(const uint8_t *tiled, int64_t n, int64_t k, const float *x, int64_t m, const float *signs1024,
                     float *y, void *ws, size_t ws_bytes, hipStream_t stream)
{
    int64_t wb, mk, mn, xb, yb;
    PTQ1_TRY(check_pq2(tiled, "tiled", n, k, signs1024 != nullptr, &wb, true));
    if (m < 0) return fail(PTQ1_ERR_SHAPE, "m = %lld is negative", (long long)m);
    if (m > kMaxGemmM) return fail(PTQ1_ERR_UNSUPPORTED, "m = %lld > %lld", (long long)m, (long long)kMaxGemmM);
    if (!mul_ok(m, k, &mk) || !mul_ok(m, n, &mn)) return fail(PTQ1_ERR_OVERFLOW, "m * k or m * n overflows");
    PTQ1_TRY(check_floats(y, "y", mn, &yb));
    if (mn == 0) return ok();
    PTQ1_TRY(check_floats(x, "x", mk, &xb));
    PTQ1_TRY(check_signs(signs1024, false));
    const ptq1::GemmPlan plan = ptq1::gemm_plan(m, n, k, true);
    const GemmWs L = gemm_layout(plan, k);
    const size_t need = L.total;
    PTQ1_TRY(check_ws(ws, ws_bytes, need, "pq2_gemm"));
    if (overlaps(y, yb, x, xb)) return fail(PTQ1_ERR_ALIAS, "y overlaps x");
    if (overlaps(y, yb, tiled, wb)) return fail(PTQ1_ERR_ALIAS, "y overlaps tiled");
    if (overlaps(ws, (int64_t)need, y, yb) || overlaps(ws, (int64_t)need, x, xb) ||
        overlaps(ws, (int64_t)need, tiled, wb))
        return fail(PTQ1_ERR_ALIAS, "ws overlaps an argument");
    char *w = static_cast<char *>(ws);
    uint16_t *xf = reinterpret_cast<uint16_t *>(w + L.frag);
    float *part = reinterpret_cast<float *>(w + L.part);
    hipError_t e = ptq1::launch_prep_frag_pq2(x, nullptr, nullptr, m, k, signs1024, 0.0f, nullptr, xf, stream);
    if (e == hipSuccess)
        e = profiled(kProfGemm, stream, [&] {
            return ptq1::launch_gemm_pq2(plan, xf, m, tiled, n, nullptr, 0, y, nullptr, nullptr, part, stream);
        });
    return hip_status(e, "pq2_gemm");
}

size_t ptq1_matvec_w2a8_workspace_bytes(int64_t n, int64_t k)
{
    if (packed_bytes(n, k) < 0) return 0;
    return lut_ws(n, 1, k);  // the split-K partials
}

ptq1_status ptq1_matvec_w2a8(const uint8_t *tiled, int64_t n, int64_t k, const float *x, const float *residual,
                             float *y, void *ws, size_t ws_bytes, hipStream_t stream)
{
    int64_t wb, xb, yb;
    PTQ1_TRY(check_matrix(tiled, "tiled", n, k, false, &wb, true));
    PTQ1_TRY(check_floats(y, "y", n, &yb));
    if (n == 0) return ok();
    if (k == 0) return fail(PTQ1_ERR_SHAPE, "k = 0");
    PTQ1_TRY(check_floats(x, "x", k, &xb));
    if (residual != nullptr) {
        int64_t rb;
        PTQ1_TRY(check_floats(residual, "residual", n, &rb));
        if (residual != y && overlaps(residual, rb, y, yb))
            return fail(PTQ1_ERR_ALIAS, "y partially overlaps residual");
    }
    const size_t need = ptq1_matvec_w2a8_workspace_bytes(n, k);
    PTQ1_TRY(check_ws(ws, ws_bytes, need, "ptq1_matvec_w2a8"));
    if (overlaps(y, yb, x, xb)) return fail(PTQ1_ERR_ALIAS, "y overlaps x");
    if (overlaps(y, yb, tiled, wb)) return fail(PTQ1_ERR_ALIAS, "y overlaps the weights");
    if (overlaps(ws, (int64_t)need, y, yb) || overlaps(ws, (int64_t)need, x, xb) ||
        overlaps(ws, (int64_t)need, tiled, wb))
        return fail(PTQ1_ERR_ALIAS, "ws overlaps an argument");
    if (residual != nullptr && overlaps(ws, (int64_t)need, residual, 4 * n))
        return fail(PTQ1_ERR_ALIAS, "ws overlaps residual");
    if (nseg_of(k) * 4 > kMaxGridY) return fail(PTQ1_ERR_UNSUPPORTED, "k = %lld too large", (long long)k);
    if (n > kMaxLutRows) return fail(PTQ1_ERR_UNSUPPORTED, "n = %lld > %lld rows", (long long)n, (long long)kMaxLutRows);
    if (wb > kMaxLutMatrixBytes) return fail(PTQ1_ERR_UNSUPPORTED, "tiled matrix above 2 GiB");
    float *part = static_cast<float *>(ws);
    hipError_t e = profiled(kProfLut1, stream, [&] {
        return ptq1::launch_matvec_lut(tiled, nullptr, 1, n, k, x, nullptr, nullptr, part, stream, true);
    });
    if (e == hipSuccess) e = ptq1::launch_lut_sum_rows(part, n, k, residual, y, stream);
    return hip_status(e, "ptq1_matvec_w2a8");
}

size_t ptq1_gemm_w2a8_workspace_bytes(int64_t m, int64_t n, int64_t k)
{
    if (packed_bytes(n, k) < 0 || m < 0 || m > kMaxGemmM) return 0;
    if (m == 0) return 0;
    return gemm_layout(ptq1::gemm_plan(m, n, k, true), k).total + round_up(static_cast<size_t>(m) * 4, kWsAlign);
}

ptq1_status ptq1_gemm_w2a8(const uint8_t *tiled, int64_t n, int64_t k, const float *x, int64_t m, float *y, void *ws,
                           size_t ws_bytes, hipStream_t stream)
{
    int64_t wb, mk, mn, xb, yb;
    PTQ1_TRY(check_matrix(tiled, "tiled", n, k, false, &wb, true));
    if (m < 0) return fail(PTQ1_ERR_SHAPE, "m = %lld is negative", (long long)m);
    if (m > kMaxGemmM) return fail(PTQ1_ERR_UNSUPPORTED, "m = %lld > %lld", (long long)m, (long long)kMaxGemmM);
    if (!mul_ok(m, k, &mk) || !mul_ok(m, n, &mn)) return fail(PTQ1_ERR_OVERFLOW, "m * k or m * n overflows");
    PTQ1_TRY(check_floats(y, "y", mn, &yb));
    if (mn == 0) return ok();
    if (k == 0) return fail(PTQ1_ERR_SHAPE, "k = 0");
    PTQ1_TRY(check_floats(x, "x", mk, &xb));
    const ptq1::GemmPlan plan = ptq1::gemm_plan(m, n, k, true);  // the int8 kernel has register-decode plans
    const GemmWs L = gemm_layout(plan, k);
    const size_t need = ptq1_gemm_w2a8_workspace_bytes(m, n, k);
    PTQ1_TRY(check_ws(ws, ws_bytes, need, "ptq1_gemm_w2a8"));
    if (overlaps(y, yb, x, xb)) return fail(PTQ1_ERR_ALIAS, "y overlaps x");
    if (overlaps(y, yb, tiled, wb)) return fail(PTQ1_ERR_ALIAS, "y overlaps tiled");
    if (overlaps(ws, (int64_t)need, y, yb) || overlaps(ws, (int64_t)need, x, xb) ||
        overlaps(ws, (int64_t)need, tiled, wb))
        return fail(PTQ1_ERR_ALIAS, "ws overlaps an argument");
    char *w = static_cast<char *>(ws);
    uint8_t *xq = reinterpret_cast<uint8_t *>(w + L.frag);  // int8 operands: m_pad * k bytes of the bf16 region
    float *part = reinterpret_cast<float *>(w + L.part);
    float *step = reinterpret_cast<float *>(w + L.total);
    hipError_t e = ptq1::launch_prep_frag_w8(x, m, k, xq, step, stream);
    if (e == hipSuccess)
        e = profiled(kProfGemm, stream, [&] {
            return ptq1::launch_gemm_i8(plan, xq, m, tiled, n, y, step, part, stream);
        });
    return hip_status(e, "ptq1_gemm_w2a8");
}

size_t pq2_ffn_workspace_bytes(int64_t m, int64_t d, int64_t f)
{
    if (m < 0 || m > kMaxGemmM || pq2_packed(f, d) < 0 || pq2_packed(d, f) < 0 || f > INT64_MAX / 2) return 0;
    if (m == 0) return 0;
    return ffn_layout(m, d, f, true).total;
}

ptq1_status pq2_ffn_block(const float *x, float *x_out, int64_t m, int64_t d, int64_t f, const uint8_t *w_gate,
                          const uint8_t *w_up, const uint8_t *w_down, const float *signs1024, float rms_eps,
                          const float *rms_gain, void *ws, size_t ws_bytes, hipStream_t stream)
{
    int64_t wgb, wub, wdb, md, xb, ob;
    if (m < 0) return fail(PTQ1_ERR_SHAPE, "m = %lld is negative", (long long)m);
    if (m > kMaxGemmM) return fail(PTQ1_ERR_UNSUPPORTED, "m = %lld > %lld", (long long)m, (long long)kMaxGemmM);
    PTQ1_TRY(check_pq2(w_gate, "w_gate", f, d, true, &wgb, true));
    PTQ1_TRY(check_pq2(w_up, "w_up", f, d, true, &wub, true));
    PTQ1_TRY(check_pq2(w_down, "w_down", d, f, true, &wdb, true));
    if (!mul_ok(m, d, &md)) return fail(PTQ1_ERR_OVERFLOW, "m * d overflows");
    PTQ1_TRY(check_floats(x_out, "x_out", md, &ob));
    if (md == 0) return ok();
    PTQ1_TRY(check_floats(x, "x", md, &xb));
    PTQ1_TRY(check_signs(signs1024, true));
    int64_t gb = 0;
    if (rms_gain != nullptr) {
        PTQ1_TRY(check_floats(rms_gain, "rms_gain", d, &gb));
        if (overlaps(x_out, ob, rms_gain, gb)) return fail(PTQ1_ERR_ALIAS, "x_out overlaps rms_gain");
    }
    if (x_out != x && overlaps(x_out, ob, x, xb)) return fail(PTQ1_ERR_ALIAS, "x_out partially overlaps x");
    if (overlaps(x_out, ob, w_gate, wgb) || overlaps(x_out, ob, w_up, wub) || overlaps(x_out, ob, w_down, wdb))
        return fail(PTQ1_ERR_ALIAS, "x_out overlaps a weight matrix");
    if (f == 0) return fail(PTQ1_ERR_SHAPE, "f = 0");
    const FfnWs L = ffn_layout(m, d, f, true);
    PTQ1_TRY(check_ws(ws, ws_bytes, L.total, "pq2_ffn_block"));
    if (overlaps(ws, (int64_t)L.total, x, xb) || overlaps(ws, (int64_t)L.total, x_out, ob))
        return fail(PTQ1_ERR_ALIAS, "ws overlaps x or x_out");
    if (rms_gain != nullptr && overlaps(ws, (int64_t)L.total, rms_gain, gb))
        return fail(PTQ1_ERR_ALIAS, "ws overlaps rms_gain");
    if (nseg_of(f) * 4 > kMaxGridY || nseg_of(d) * 4 > kMaxGridY)
        return fail(PTQ1_ERR_UNSUPPORTED, "d or f too large");
    if (m == 1 && (f > kMaxLutRows || d > kMaxLutRows))
        return fail(PTQ1_ERR_UNSUPPORTED, "d or f > %lld rows", (long long)kMaxLutRows);
    if (m == 1 && (wgb > kMaxLutMatrixBytes || wub > kMaxLutMatrixBytes || wdb > kMaxLutMatrixBytes))
        return fail(PTQ1_ERR_UNSUPPORTED, "tiled matrices above 2 GiB");
    char *w = static_cast<char *>(ws);
    hipError_t e;
    if (m == 1) {
        // the PTQ1_0 block's composition over the PQ2_0 lookup kernel
        float *part = reinterpret_cast<float *>(w + L.part);
        float *h = reinterpret_cast<float *>(w + L.hr);
        e = profiled(kProfPq2, stream, [&] {
            return ptq1::launch_pq2_matvec(w_gate, w_up, 2, f, d, x, signs1024, rms_gain, part, stream);
        });
        if (e == hipSuccess)
            e = ptq1::launch_lut_gate_up_sum(part, f, d, rms_eps > 0.0f ? x : nullptr, d, rms_eps, nullptr, nullptr,
                                             h, stream);
        if (e == hipSuccess)
            e = profiled(kProfPq2, stream, [&] {
                return ptq1::launch_pq2_matvec(w_down, nullptr, 1, d, f, h, signs1024, nullptr, part, stream);
            });
        if (e == hipSuccess) e = ptq1::launch_lut_sum_rows(part, d, f, x, x_out, stream);
    } else {
        uint16_t *xf = reinterpret_cast<uint16_t *>(w + L.xb);
        float *g = reinterpret_cast<float *>(w + L.g);
        float *u = reinterpret_cast<float *>(w + L.u);
        float *part = reinterpret_cast<float *>(w + L.part);
        const bool fold = ptq1::gemm_fold_ok(L.gu);  // as in ptq1_ffn_block
        e = ptq1::launch_prep_frag_pq2(x, nullptr, nullptr, m, d, signs1024, rms_eps, rms_gain, xf, stream);
        if (e == hipSuccess)
            e = profiled(kProfGemm, stream, [&] {
                return ptq1::launch_gemm_pq2(L.gu, xf, m, w_gate, f, w_up, f, g, u, nullptr, part, stream, !fold);
            });
        if (e == hipSuccess)
            e = ptq1::launch_prep_frag_pq2(nullptr, g, u, m, f, signs1024, 0.0f, nullptr, xf, stream,
                                           fold ? ptq1::gemm_sk_view(L.gu, part) : ptq1::SkView{});
        if (e == hipSuccess)
            e = profiled(kProfGemm, stream, [&] {
                return ptq1::launch_gemm_pq2(L.dn, xf, m, w_down, d, nullptr, 0, x_out, nullptr, x, part, stream);
            });
    }
    return hip_status(e, "pq2_ffn_block");
}

}  // extern "C"
