// api.cpp -- the C ABI declared in include/pagedattn.h: host-side argument
// checks, error reporting, workspace sizing and dispatch to the kernels.
//
// Every check runs before anything is enqueued; a failing call writes
// nothing and leaves a message naming the argument ("Radiance Architecture
// Plugins -- declaring a model", section "Step: issuing the graph": zero rows
// is a shape error that writes nothing; a failing helper sets a named
// status).  Unserved shapes are refused, never routed elsewhere (same page,
// section "Probe: what the plugin measured").
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/pagedattn.h"
#include "kernels.h"

namespace pa {
int split_tiles(int rows, int g);
}

namespace {

thread_local char t_err[256] = "";
thread_local hipEvent_t t_ev_start = nullptr;
thread_local hipEvent_t t_ev_stop = nullptr;
std::atomic<int32_t> g_max_workgroups{0};

// The mixed step's second stream and compute-unit count, per device, made
// on first use with that device current and kept until the process ends;
// and each thread's fork / join events per device.
std::mutex g_side_mu;
hipStream_t g_side[pa::kMaxDevices];
int g_cus[pa::kMaxDevices];
thread_local hipEvent_t t_fork[pa::kMaxDevices];
thread_local hipEvent_t t_join[pa::kMaxDevices];

hipError_t side_stream(hipStream_t* side, int* cus, hipEvent_t* fork, hipEvent_t* join)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= pa::kMaxDevices)
        return hipErrorInvalidDevice;
    {
        std::lock_guard<std::mutex> lock(g_side_mu);
        if (!g_side[dev]) {
            int n = 0;
            e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
            if (e != hipSuccess)
                return e;
            hipStream_t st = nullptr;
            e = hipStreamCreateWithFlags(&st, hipStreamNonBlocking);
            if (e != hipSuccess)
                return e;
            g_cus[dev] = n;
            g_side[dev] = st;
        }
        *side = g_side[dev];
        *cus = g_cus[dev];
    }
    for (hipEvent_t* ev : {&t_fork[dev], &t_join[dev]}) {
        if (!*ev) {
            e = hipEventCreateWithFlags(ev, hipEventDisableTiming);
            if (e != hipSuccess)
                return e;
        }
    }
    *fork = t_fork[dev];
    *join = t_join[dev];
    return hipSuccess;
}

int fail(int code, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(t_err, sizeof t_err, fmt, ap);
    va_end(ap);
    return code;
}

int ok()
{
    t_err[0] = 0;
    return ATTN_OK;
}

int from_hip(hipError_t e, const char* what)
{
    if (e == hipSuccess)
        return ok();
    if (e == hipErrorNotSupported)
        return fail(ATTN_E_UNSUPPORTED, "%s: shape not served by the kernels", what);
    return fail(ATTN_E_DEVICE, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

bool head_dim_ok(int32_t d) { return d == 128 || d == 256; }

// Checks common to decode / verify / prefill.  Returns ATTN_OK or a code.
int check_common(const char* fn, const void* q, const void* k_pool, const void* v_pool,
                 const float* k_scale, const float* v_scale, int64_t n_pages,
                 const int32_t* block_table, int32_t max_pages, int32_t n_head,
                 int32_t n_head_kv, int32_t head_dim, int32_t page_size, attn_kv_dtype kv_dtype,
                 const void* out)
{
    if (!q)
        return fail(ATTN_E_ARG, "%s: q is NULL", fn);
    if (!k_pool || !v_pool)
        return fail(ATTN_E_ARG, "%s: k_pool/v_pool is NULL", fn);
    if (!block_table)
        return fail(ATTN_E_ARG, "%s: block_table is NULL", fn);
    if (!out)
        return fail(ATTN_E_ARG, "%s: out is NULL", fn);
    if (kv_dtype != ATTN_KV_BF16 && kv_dtype != ATTN_KV_FP8_E4M3)
        return fail(ATTN_E_ARG, "%s: kv_dtype %d is not a kv dtype", fn, (int)kv_dtype);
    if (kv_dtype == ATTN_KV_FP8_E4M3 && (!k_scale || !v_scale))
        return fail(ATTN_E_ARG, "%s: fp8 kv needs k_scale and v_scale", fn);
    if (kv_dtype == ATTN_KV_BF16 && (k_scale || v_scale))
        return fail(ATTN_E_ARG, "%s: bf16 kv takes no scales (pass NULL)", fn);
    if (n_pages <= 0)
        return fail(ATTN_E_SHAPE, "%s: n_pages must be positive (got %lld)", fn,
                    (long long)n_pages);
    if (n_pages > (int64_t)INT32_MAX)
        return fail(ATTN_E_UNSUPPORTED, "%s: n_pages above 2^31-1", fn);
    if (max_pages <= 0)
        return fail(ATTN_E_SHAPE, "%s: max_pages_per_seq must be positive (got %d)", fn,
                    max_pages);
    if ((int64_t)max_pages * ATTN_PAGE_SIZE > (int64_t)INT32_MAX)
        return fail(ATTN_E_UNSUPPORTED, "%s: max_pages_per_seq too large", fn);
    if (n_head <= 0 || n_head_kv <= 0)
        return fail(ATTN_E_SHAPE, "%s: n_head (%d) and n_head_kv (%d) must be positive", fn,
                    n_head, n_head_kv);
    if (n_head % n_head_kv != 0)
        return fail(ATTN_E_SHAPE, "%s: n_head (%d) is not a multiple of n_head_kv (%d)", fn,
                    n_head, n_head_kv);
    if (head_dim <= 0)
        return fail(ATTN_E_SHAPE, "%s: head_dim must be positive (got %d)", fn, head_dim);
    if (!head_dim_ok(head_dim))
        return fail(ATTN_E_UNSUPPORTED, "%s: head_dim %d not served (128, 256)", fn, head_dim);
    if (page_size != ATTN_PAGE_SIZE)
        return fail(ATTN_E_UNSUPPORTED, "%s: page_size %d not served (16)", fn, page_size);
    // The kernels address the per-page scale arrays through one bounds-checked
    // buffer resource each, which spans less than 2 GiB.
    if (n_pages * (int64_t)n_head_kv * 4 >= ((int64_t)1 << 31))
        return fail(ATTN_E_UNSUPPORTED, "%s: n_pages * n_head_kv above 2^29", fn);
    return ATTN_OK;
}

int check_workspace(const char* fn, void* ws, size_t have, size_t need)
{
    if (need == 0)
        return ATTN_OK;
    if (!ws)
        return fail(ATTN_E_WORKSPACE, "%s: workspace is NULL (%zu bytes needed)", fn, need);
    if (((uintptr_t)ws & 255u) != 0)
        return fail(ATTN_E_WORKSPACE, "%s: workspace must be 256-byte aligned", fn);
    if (have < need)
        return fail(ATTN_E_WORKSPACE, "%s: workspace has %zu bytes, %zu needed", fn, have, need);
    return ATTN_OK;
}

size_t split_ws_bytes(int32_t rows, int32_t n_seq, int32_t max_pages, int32_t n_head,
                      int32_t head_dim)
{
    const int64_t ms = pa::max_splits(max_pages, ATTN_PAGE_SIZE);
    const int64_t rec = (int64_t)n_seq * ms * rows * n_head;
    int64_t o_bytes = rec * head_dim * 4;
    o_bytes = (o_bytes + 255) / 256 * 256;
    return (size_t)(o_bytes + rec * 2 * 4);
}

// Workspace of a tree round: the branch views' table rows, lengths and
// floors, then the split-K partials of n_seq * 8 one-row sequences.
size_t tree_ws_bytes(int32_t n_seq, int32_t max_pages, int32_t n_head, int32_t head_dim,
                     size_t* off_lens, size_t* off_floor, size_t* off_split)
{
    const int64_t nv = (int64_t)n_seq * ATTN_VERIFY_ROWS;
    const size_t tb = (size_t)((nv * max_pages * 4 + 255) / 256 * 256);
    const size_t lb = (size_t)((nv * 4 + 255) / 256 * 256);
    if (off_lens)
        *off_lens = tb;
    if (off_floor)
        *off_floor = tb + lb;
    if (off_split)
        *off_split = tb + 2 * lb;
    return tb + 2 * lb + split_ws_bytes(1, (int32_t)nv, max_pages, n_head, head_dim);
}


// Host checks of a decode / verify call and its kernel arguments; enqueues
// nothing.
int split_setup(pa::SplitArgs& a, const char* fn, int32_t rows, const void* q,
                const void* k_pool, const void* v_pool, const float* k_scale,
                const float* v_scale, int64_t n_pages, const int32_t* block_table,
                int32_t max_pages, const int32_t* ctx_lens, int32_t n_seq, int32_t n_head,
                int32_t n_head_kv, int32_t head_dim, int32_t page_size, attn_kv_dtype kv_dtype,
                void* out, void* workspace, size_t workspace_bytes, int32_t window,
                const int32_t* kv_floor, int below_round, int phase, bool noalloc)
{
    int rc = check_common(fn, q, k_pool, v_pool, k_scale, v_scale, n_pages, block_table,
                          max_pages, n_head, n_head_kv, head_dim, page_size, kv_dtype, out);
    if (rc != ATTN_OK)
        return rc;
    if (!ctx_lens)
        return fail(ATTN_E_ARG, "%s: ctx_lens is NULL", fn);
    if (n_seq <= 0)
        return fail(ATTN_E_SHAPE, "%s: zero sequences is not a call (n_seq = %d)", fn, n_seq);
    if (n_seq > pa::kMaxSeq)
        return fail(ATTN_E_UNSUPPORTED, "%s: n_seq %d above %d", fn, n_seq, pa::kMaxSeq);
    const int g = n_head / n_head_kv;
    if (g > 16)
        return fail(ATTN_E_UNSUPPORTED, "%s: %d query heads per kv head (at most 16)", fn, g);
    // One sequence's query rows, and one split's partial outputs, are each
    // addressed through a buffer resource spanning less than 2 GiB.
    if ((int64_t)rows * n_head * head_dim * 4 >= ((int64_t)1 << 31))
        return fail(ATTN_E_UNSUPPORTED, "%s: rows * n_head * head_dim too large", fn);
    // A split's partials span its rows' records, max_split * n_head apart.
    const int64_t ms = pa::max_splits(max_pages, ATTN_PAGE_SIZE);
    if (((int64_t)(rows - 1) * ms * n_head + n_head) * head_dim * 4 >= ((int64_t)1 << 31))
        return fail(ATTN_E_UNSUPPORTED, "%s: rows x splits x heads too large", fn);
    const size_t need = split_ws_bytes(rows, n_seq, max_pages, n_head, head_dim);
    if (noalloc) {
        // The partials go to the library's per-device scratch array.
        if (need > pa::kScratchBytes)
            return fail(ATTN_E_WORKSPACE,
                        "%s: the call needs %zu bytes of split partials; the scratch array "
                        "holds %zu (call attn_paged_decode with a workspace)",
                        fn, need, pa::kScratchBytes);
        rc = from_hip(pa::scratch_address(&workspace), fn);
        if (rc != ATTN_OK)
            return rc;
        workspace_bytes = pa::kScratchBytes;
    }
    rc = check_workspace(fn, workspace, workspace_bytes, need);
    if (rc != ATTN_OK)
        return rc;

    a.q = q;
    a.k_pool = k_pool;
    a.v_pool = v_pool;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    a.n_pages = n_pages;
    a.block_table = block_table;
    a.max_pages = max_pages;
    a.ctx_lens = ctx_lens;
    a.n_seq = n_seq;
    a.n_head = n_head;
    a.n_head_kv = n_head_kv;
    a.head_dim = head_dim;
    a.rows = rows;
    a.fp8 = kv_dtype == ATTN_KV_FP8_E4M3;
    a.out = out;
    a.max_split = (int32_t)pa::max_splits(max_pages, ATTN_PAGE_SIZE);
    const int64_t rec = (int64_t)n_seq * a.max_split * rows * n_head;
    const int64_t o_bytes = (rec * head_dim * 4 + 255) / 256 * 256;
    a.o_part = (float*)workspace;
    a.ml_part = (float*)((char*)workspace + o_bytes);
    a.ev_start = t_ev_start;
    a.ev_stop = t_ev_stop;
    t_ev_start = t_ev_stop = nullptr;
    a.max_blocks = g_max_workgroups.load(std::memory_order_relaxed);
    a.window = window;
    a.kv_floor = kv_floor;
    a.below_round = below_round;
    a.phase = phase;
    return ATTN_OK;
}

int split_call(const char* fn, int32_t rows, const void* q, const void* k_pool,
               const void* v_pool, const float* k_scale, const float* v_scale, int64_t n_pages,
               const int32_t* block_table, int32_t max_pages, const int32_t* ctx_lens,
               int32_t n_seq, int32_t n_head, int32_t n_head_kv, int32_t head_dim,
               int32_t page_size, attn_kv_dtype kv_dtype, void* out, void* workspace,
               size_t workspace_bytes, hipStream_t stream, int32_t window = 0,
               const int32_t* kv_floor = nullptr, int below_round = 0, int phase = 0,
               bool noalloc = false)
{
    pa::SplitArgs a;
    const int rc = split_setup(a, fn, rows, q, k_pool, v_pool, k_scale, v_scale, n_pages,
                               block_table, max_pages, ctx_lens, n_seq, n_head, n_head_kv,
                               head_dim, page_size, kv_dtype, out, workspace, workspace_bytes,
                               window, kv_floor, below_round, phase, noalloc);
    if (rc != ATTN_OK)
        return rc;
    return from_hip(pa::launch_split_decode(a, stream), fn);
}

}  // namespace

namespace pa {
int set_error(int code, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(t_err, sizeof t_err, fmt, ap);
    va_end(ap);
    return code;
}
int clear_error() { return ok(); }
}  // namespace pa

extern "C" {

const char* attn_last_error(void) { return t_err; }

int attn_check_device(const int32_t* block_table, const int32_t* ctx_lens,
                      const int32_t* kv_floor, int32_t window, int32_t n_seq, int32_t rows,
                      int32_t max_pages_per_seq, int32_t page_size, int64_t n_pages,
                      int64_t* err_word, hipStream_t stream)
{
    const char* fn = "attn_check_device";
    if (!block_table || !ctx_lens || !err_word)
        return fail(ATTN_E_ARG, "%s: block_table, ctx_lens and err_word must not be NULL", fn);
    if (n_seq <= 0 || rows <= 0)
        return fail(ATTN_E_SHAPE, "%s: zero sequences or rows is not a call (%d, %d)", fn, n_seq,
                    rows);
    if (max_pages_per_seq <= 0 || n_pages <= 0)
        return fail(ATTN_E_SHAPE, "%s: max_pages_per_seq and n_pages must be positive", fn);
    if (page_size != ATTN_PAGE_SIZE)
        return fail(ATTN_E_UNSUPPORTED, "%s: page_size %d not served", fn, page_size);
    if (window < 0)
        return fail(ATTN_E_RANGE, "%s: window %d is negative", fn, window);
    pa::CheckArgs a;
    a.block_table = block_table;
    a.ctx_lens = ctx_lens;
    a.kv_floor = kv_floor;
    a.window = window;
    a.n_seq = n_seq;
    a.rows = rows;
    a.max_pages = max_pages_per_seq;
    a.page_size = page_size;
    a.n_pages = n_pages;
    a.err = err_word;
    return from_hip(pa::launch_check(a, stream), fn);
}

void attn_set_kernel_timer(hipEvent_t start, hipEvent_t stop)
{
    t_ev_start = start;
    t_ev_stop = stop;
}

void attn_set_max_workgroups(int32_t n)
{
    g_max_workgroups.store(n > 0 ? n : 0, std::memory_order_relaxed);
}

int attn_caps(int32_t head_dim, int32_t page_size, attn_kv_dtype kv_dtype)
{
    if (kv_dtype != ATTN_KV_BF16 && kv_dtype != ATTN_KV_FP8_E4M3)
        return fail(ATTN_E_UNSUPPORTED, "attn_caps: kv_dtype %d unknown", (int)kv_dtype);
    if (!head_dim_ok(head_dim))
        return fail(ATTN_E_UNSUPPORTED, "attn_caps: head_dim %d not served", head_dim);
    if (page_size != ATTN_PAGE_SIZE)
        return fail(ATTN_E_UNSUPPORTED, "attn_caps: page_size %d not served", page_size);
    return ok();
}

size_t attn_paged_workspace_bytes(int op, int32_t n_seq, int32_t max_pages_per_seq,
                                  int32_t n_head, int32_t head_dim)
{
    if (n_seq <= 0 || max_pages_per_seq <= 0 || n_head <= 0 || !head_dim_ok(head_dim))
        return 0;
    switch (op) {
    case 0: return split_ws_bytes(1, n_seq, max_pages_per_seq, n_head, head_dim);
    case 1: return split_ws_bytes(ATTN_VERIFY_ROWS, n_seq, max_pages_per_seq, n_head, head_dim);
    case 2: return 0;
    case 3: return split_ws_bytes(1, n_seq, max_pages_per_seq, n_head, head_dim);
    case 4:
        return tree_ws_bytes(n_seq, max_pages_per_seq, n_head, head_dim, nullptr, nullptr,
                             nullptr);
    default: return 0;
    }
}

int attn_paged_decode(const void* q, const void* k_pool, const void* v_pool,
                      const float* k_scale, const float* v_scale, int64_t n_pages,
                      const int32_t* block_table, int32_t max_pages_per_seq,
                      const int32_t* ctx_lens, int32_t n_seq, int32_t n_head,
                      int32_t n_head_kv, int32_t head_dim, int32_t page_size,
                      attn_kv_dtype kv_dtype, void* out, void* workspace,
                      size_t workspace_bytes, hipStream_t stream)
{
    return split_call("attn_paged_decode", 1, q, k_pool, v_pool, k_scale, v_scale, n_pages,
                      block_table, max_pages_per_seq, ctx_lens, n_seq, n_head, n_head_kv,
                      head_dim, page_size, kv_dtype, out, workspace, workspace_bytes, stream);
}

int attn_paged_decode_noalloc(const void* q, const void* k_pool, const void* v_pool,
                              const float* k_scale, const float* v_scale, int64_t n_pages,
                              const int32_t* block_table, int32_t max_pages_per_seq,
                              const int32_t* ctx_lens, int32_t n_seq, int32_t n_head,
                              int32_t n_head_kv, int32_t head_dim, int32_t page_size,
                              attn_kv_dtype kv_dtype, void* out, hipStream_t stream)
{
    return split_call("attn_paged_decode_noalloc", 1, q, k_pool, v_pool, k_scale, v_scale,
                      n_pages, block_table, max_pages_per_seq, ctx_lens, n_seq, n_head,
                      n_head_kv, head_dim, page_size, kv_dtype, out, nullptr, 0, stream, 0,
                      nullptr, 0, 0, true);
}

int attn_paged_verify(const void* q, const void* k_pool, const void* v_pool,
                      const float* k_scale, const float* v_scale, int64_t n_pages,
                      const int32_t* block_table, int32_t max_pages_per_seq,
                      const int32_t* ctx_lens, int32_t n_seq, int32_t n_head,
                      int32_t n_head_kv, int32_t head_dim, int32_t page_size,
                      attn_kv_dtype kv_dtype, void* out, void* workspace,
                      size_t workspace_bytes, hipStream_t stream)
{
    return split_call("attn_paged_verify", ATTN_VERIFY_ROWS, q, k_pool, v_pool, k_scale,
                      v_scale, n_pages, block_table, max_pages_per_seq, ctx_lens, n_seq, n_head,
                      n_head_kv, head_dim, page_size, kv_dtype, out, workspace, workspace_bytes,
                      stream);
}

int attn_paged_verify_width(const void* q, const void* k_pool, const void* v_pool,
                            const float* k_scale, const float* v_scale, int64_t n_pages,
                            const int32_t* block_table, int32_t max_pages_per_seq,
                            const int32_t* ctx_lens, int32_t n_seq, int32_t width,
                            int32_t n_head, int32_t n_head_kv, int32_t head_dim,
                            int32_t page_size, attn_kv_dtype kv_dtype, void* out,
                            void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    const char* fn = "attn_paged_verify_width";
    if (width <= 0)
        return fail(ATTN_E_SHAPE, "%s: zero rows is not a call (width = %d)", fn, width);
    if (width > ATTN_VERIFY_ROWS)
        return fail(ATTN_E_UNSUPPORTED, "%s: width %d above %d", fn, width, ATTN_VERIFY_ROWS);
    return split_call(fn, width, q, k_pool, v_pool, k_scale, v_scale, n_pages, block_table,
                      max_pages_per_seq, ctx_lens, n_seq, n_head, n_head_kv, head_dim, page_size,
                      kv_dtype, out, workspace, workspace_bytes, stream);
}

static int prefill_call(const char* fn, const void* q, int32_t n_rows, const void* k_pool,
                        const void* v_pool, const float* k_scale, const float* v_scale,
                        int64_t n_pages, const int32_t* block_table, int32_t max_pages_per_seq,
                        int32_t ctx_len, int32_t window, int32_t kv_floor, int32_t n_head,
                        int32_t n_head_kv, int32_t head_dim, int32_t page_size,
                        attn_kv_dtype kv_dtype, void* out, hipStream_t stream,
                        int32_t prefill_fp8 = 0)
{
    int rc = check_common(fn, q, k_pool, v_pool, k_scale, v_scale, n_pages, block_table,
                          max_pages_per_seq, n_head, n_head_kv, head_dim, page_size, kv_dtype,
                          out);
    if (rc != ATTN_OK)
        return rc;
    if (prefill_fp8 & ~(ATTN_PREFILL_FP8_QK | ATTN_PREFILL_FP8_PV))
        return fail(ATTN_E_UNSUPPORTED,
                    "%s: prefill_fp8 bits 0x%x (only ATTN_PREFILL_FP8_QK, ATTN_PREFILL_FP8_PV)", fn,
                    (unsigned)prefill_fp8);
    if (prefill_fp8 && kv_dtype != ATTN_KV_FP8_E4M3)
        return fail(ATTN_E_UNSUPPORTED, "%s: prefill_fp8 bits need an fp8 cache", fn);
    if (n_rows <= 0)
        return fail(ATTN_E_SHAPE, "%s: zero rows is not a call (n_rows = %d)", fn, n_rows);
    if (ctx_len < n_rows)
        return fail(ATTN_E_RANGE, "%s: ctx_len %d is below n_rows %d", fn, ctx_len, n_rows);
    if ((int64_t)ctx_len > (int64_t)max_pages_per_seq * page_size)
        return fail(ATTN_E_RANGE, "%s: ctx_len %d exceeds max_pages_per_seq * page_size", fn,
                    ctx_len);
    if (window < 0)
        return fail(ATTN_E_RANGE, "%s: window %d is negative", fn, window);
    if (kv_floor < 0 || kv_floor > ctx_len - n_rows)
        return fail(ATTN_E_RANGE, "%s: kv_floor %d outside 0 .. ctx_len - n_rows (%d)", fn,
                    kv_floor, ctx_len - n_rows);
    pa::PrefillArgs a;
    a.q = q;
    a.n_rows = n_rows;
    a.k_pool = k_pool;
    a.v_pool = v_pool;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    a.n_pages = n_pages;
    a.block_table = block_table;
    a.max_pages = max_pages_per_seq;
    a.ctx_len = ctx_len;
    a.n_head = n_head;
    a.n_head_kv = n_head_kv;
    a.head_dim = head_dim;
    a.fp8 = kv_dtype == ATTN_KV_FP8_E4M3;
    a.out = out;
    a.ev_start = t_ev_start;
    a.ev_stop = t_ev_stop;
    t_ev_start = t_ev_stop = nullptr;
    a.cu_seqlens = nullptr;
    a.ctx_lens = nullptr;
    a.n_var = 1;
    a.max_q_len = n_rows;
    a.n_tok = n_rows;
    a.window = window;
    a.kv_floor = kv_floor;
    a.qk_fp8 = (prefill_fp8 & ATTN_PREFILL_FP8_QK) != 0;
    a.pv_fp8 = (prefill_fp8 & ATTN_PREFILL_FP8_PV) != 0;
    return from_hip(pa::launch_prefill(a, stream), fn);
}

int attn_paged_verify_tree(const void* q, void* k_pool, void* v_pool, float* k_scale,
                           float* v_scale, int64_t n_pages, const int32_t* block_table,
                           int32_t max_pages_per_seq, const int32_t* ctx_lens, int32_t n_seq,
                           int32_t width, const int32_t* tree_mask, const int32_t* scratch_pages,
                           int32_t n_head, int32_t n_head_kv, int32_t head_dim,
                           int32_t page_size, attn_kv_dtype kv_dtype, void* out,
                           void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    const char* fn = "attn_paged_verify_tree";
    int rc = check_common(fn, q, k_pool, v_pool, k_scale, v_scale, n_pages, block_table,
                          max_pages_per_seq, n_head, n_head_kv, head_dim, page_size, kv_dtype,
                          out);
    if (rc != ATTN_OK)
        return rc;
    if (!ctx_lens || !tree_mask || !scratch_pages)
        return fail(ATTN_E_ARG, "%s: ctx_lens, tree_mask and scratch_pages must not be NULL",
                    fn);
    if (width <= 0)
        return fail(ATTN_E_SHAPE, "%s: zero rows is not a call (width = %d)", fn, width);
    if (width > ATTN_VERIFY_ROWS)
        return fail(ATTN_E_UNSUPPORTED, "%s: width %d above %d", fn, width, ATTN_VERIFY_ROWS);
    if (n_seq <= 0)
        return fail(ATTN_E_SHAPE, "%s: zero sequences is not a call (n_seq = %d)", fn, n_seq);
    if ((int64_t)n_seq * width > pa::kMaxSeq)
        return fail(ATTN_E_UNSUPPORTED, "%s: n_seq * width %lld above %d", fn,
                    (long long)n_seq * width, pa::kMaxSeq);
    if (n_head / n_head_kv > 16)
        return fail(ATTN_E_UNSUPPORTED, "%s: %d query heads per kv head (at most 16)", fn,
                    n_head / n_head_kv);
    size_t off_lens = 0, off_floor = 0, off_split = 0;
    const size_t need = tree_ws_bytes(n_seq, max_pages_per_seq, n_head, head_dim, &off_lens,
                                      &off_floor, &off_split);
    rc = check_workspace(fn, workspace, workspace_bytes, need);
    if (rc != ATTN_OK)
        return rc;
    pa::TreeArgs t;
    t.block_table = block_table;
    t.ctx_lens = ctx_lens;
    t.tree_mask = tree_mask;
    t.scratch = scratch_pages;
    t.k_pool = k_pool;
    t.v_pool = v_pool;
    t.k_scale = k_scale;
    t.v_scale = v_scale;
    t.n_pages = n_pages;
    t.n_seq = n_seq;
    t.rows = width;
    t.max_pages = max_pages_per_seq;
    t.n_head_kv = n_head_kv;
    t.head_dim = head_dim;
    t.fp8 = kv_dtype == ATTN_KV_FP8_E4M3;
    t.vtable = (int32_t*)workspace;
    t.vlens = (int32_t*)((char*)workspace + off_lens);
    t.vfloor = (int32_t*)((char*)workspace + off_floor);
    t.chunk = pa::decode_chunk(head_dim, kv_dtype == ATTN_KV_FP8_E4M3);
    // Each (sequence, row) is a one-row decode over its branch view, in
    // three launches that keep that arithmetic: (A) the splits wholly below
    // the one holding C0 = ctx_len - width hold context only, the same keys
    // for every row, so the round's split kernel computes them for all rows
    // at once (a round row's arithmetic is the decode row's); (B) the split
    // holding C0 and the next differ per branch: the one-row split kernel
    // over the views, from the first key of C0's split; (C) the combine of
    // each view over all its splits.  A and B write the same partial records
    // ((sequence, row) = view, split, head).  The checks of the three calls
    // were made above or hold by construction.
    // Shapes the round's split kernel does not serve take the plain decode of
    // every view over all its splits (one launch, the same bits).
    void* ws = (char*)workspace + off_split;
    const size_t wsb = workspace_bytes - off_split;
    const int64_t ms = pa::max_splits(max_pages_per_seq, ATTN_PAGE_SIZE);
    const bool shared =
        ((int64_t)(width - 1) * ms * n_head + n_head) * head_dim * 4 < ((int64_t)1 << 31);
    rc = from_hip(pa::launch_tree_stage(t, stream), fn);
    if (rc != ATTN_OK)
        return rc;
    if (!shared)
        return split_call(fn, 1, q, k_pool, v_pool, k_scale, v_scale, n_pages, t.vtable,
                          max_pages_per_seq, t.vlens, n_seq * width, n_head, n_head_kv,
                          head_dim, page_size, kv_dtype, out, ws, wsb, stream);
    rc = split_call(fn, width, q, k_pool, v_pool, k_scale, v_scale, n_pages, block_table,
                    max_pages_per_seq, ctx_lens, n_seq, n_head, n_head_kv, head_dim, page_size,
                    kv_dtype, out, ws, wsb, stream, 0, nullptr, 1, 1);
    if (rc != ATTN_OK)
        return rc;
    rc = split_call(fn, 1, q, k_pool, v_pool, k_scale, v_scale, n_pages, t.vtable,
                    max_pages_per_seq, t.vlens, n_seq * width, n_head, n_head_kv, head_dim,
                    page_size, kv_dtype, out, ws, wsb, stream, 0, t.vfloor, 0, 1);
    if (rc != ATTN_OK)
        return rc;
    return split_call(fn, 1, q, k_pool, v_pool, k_scale, v_scale, n_pages, t.vtable,
                      max_pages_per_seq, t.vlens, n_seq * width, n_head, n_head_kv, head_dim,
                      page_size, kv_dtype, out, ws, wsb, stream, 0, nullptr, 0, 2);
}

int attn_paged_prefill(const void* q, int32_t n_rows, const void* k_pool, const void* v_pool,
                       const float* k_scale, const float* v_scale, int64_t n_pages,
                       const int32_t* block_table, int32_t max_pages_per_seq, int32_t ctx_len,
                       int32_t n_head, int32_t n_head_kv, int32_t head_dim, int32_t page_size,
                       attn_kv_dtype kv_dtype, void* out, void* workspace,
                       size_t workspace_bytes, hipStream_t stream)
{
    (void)workspace;
    (void)workspace_bytes;
    return prefill_call("attn_paged_prefill", q, n_rows, k_pool, v_pool, k_scale, v_scale,
                        n_pages, block_table, max_pages_per_seq, ctx_len, 0, 0, n_head,
                        n_head_kv, head_dim, page_size, kv_dtype, out, stream);
}

int attn_paged_prefill_fp8(const void* q, int32_t n_rows, const void* k_pool,
                           const void* v_pool, const float* k_scale, const float* v_scale,
                           int64_t n_pages, const int32_t* block_table,
                           int32_t max_pages_per_seq, int32_t ctx_len, int32_t n_head,
                           int32_t n_head_kv, int32_t head_dim, int32_t page_size,
                           attn_kv_dtype kv_dtype, int32_t prefill_fp8, void* out,
                           void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    (void)workspace;
    (void)workspace_bytes;
    return prefill_call("attn_paged_prefill_fp8", q, n_rows, k_pool, v_pool, k_scale, v_scale,
                        n_pages, block_table, max_pages_per_seq, ctx_len, 0, 0, n_head,
                        n_head_kv, head_dim, page_size, kv_dtype, out, stream, prefill_fp8);
}

int attn_paged_prefill_window(const void* q, int32_t n_rows, const void* k_pool,
                              const void* v_pool, const float* k_scale, const float* v_scale,
                              int64_t n_pages, const int32_t* block_table,
                              int32_t max_pages_per_seq, int32_t ctx_len, int32_t window,
                              int32_t kv_floor, int32_t n_head, int32_t n_head_kv,
                              int32_t head_dim, int32_t page_size, attn_kv_dtype kv_dtype,
                              void* out, void* workspace, size_t workspace_bytes,
                              hipStream_t stream)
{
    (void)workspace;
    (void)workspace_bytes;
    return prefill_call("attn_paged_prefill_window", q, n_rows, k_pool, v_pool, k_scale, v_scale,
                        n_pages, block_table, max_pages_per_seq, ctx_len, window, kv_floor,
                        n_head, n_head_kv, head_dim, page_size, kv_dtype, out, stream);
}

int attn_paged_decode_window(const void* q, int32_t rows, const void* k_pool,
                             const void* v_pool, const float* k_scale, const float* v_scale,
                             int64_t n_pages, const int32_t* block_table,
                             int32_t max_pages_per_seq, const int32_t* ctx_lens, int32_t n_seq,
                             int32_t window, const int32_t* kv_floor, int32_t n_head,
                             int32_t n_head_kv, int32_t head_dim, int32_t page_size,
                             attn_kv_dtype kv_dtype, void* out, void* workspace,
                             size_t workspace_bytes, hipStream_t stream)
{
    const char* fn = "attn_paged_decode_window";
    if (rows <= 0)
        return fail(ATTN_E_SHAPE, "%s: zero rows is not a call (rows = %d)", fn, rows);
    if (rows > ATTN_VERIFY_ROWS)
        return fail(ATTN_E_UNSUPPORTED, "%s: rows %d above %d", fn, rows, ATTN_VERIFY_ROWS);
    if (window < 0)
        return fail(ATTN_E_RANGE, "%s: window %d is negative", fn, window);
    return split_call(fn, rows, q, k_pool, v_pool, k_scale, v_scale, n_pages, block_table,
                      max_pages_per_seq, ctx_lens, n_seq, n_head, n_head_kv, head_dim, page_size,
                      kv_dtype, out, workspace, workspace_bytes, stream, window, kv_floor);
}

int attn_paged_mixed(const void* q, int32_t n_tok, const int32_t* cu_seqlens, int32_t n_seq,
                     int32_t n_seq_decode, int32_t max_q_len, const void* k_pool,
                     const void* v_pool, const float* k_scale, const float* v_scale,
                     int64_t n_pages, const int32_t* block_table, int32_t max_pages_per_seq,
                     const int32_t* ctx_lens, int32_t n_head, int32_t n_head_kv,
                     int32_t head_dim, int32_t page_size, attn_kv_dtype kv_dtype, void* out,
                     void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    const char* fn = "attn_paged_mixed";
    int rc = check_common(fn, q, k_pool, v_pool, k_scale, v_scale, n_pages, block_table,
                          max_pages_per_seq, n_head, n_head_kv, head_dim, page_size, kv_dtype,
                          out);
    if (rc != ATTN_OK)
        return rc;
    if (!ctx_lens)
        return fail(ATTN_E_ARG, "%s: ctx_lens is NULL", fn);
    if (n_tok <= 0)
        return fail(ATTN_E_SHAPE, "%s: zero rows is not a call (n_tok = %d)", fn, n_tok);
    if (n_seq <= 0)
        return fail(ATTN_E_SHAPE, "%s: zero sequences is not a call (n_seq = %d)", fn, n_seq);
    if (n_seq_decode < 0 || n_seq_decode > n_seq)
        return fail(ATTN_E_SHAPE, "%s: n_seq_decode %d outside 0 .. n_seq (%d)", fn,
                    n_seq_decode, n_seq);
    const int32_t n_chunk = n_seq - n_seq_decode;
    if (n_chunk > 0) {
        if (!cu_seqlens)
            return fail(ATTN_E_ARG, "%s: cu_seqlens is NULL", fn);
        if (n_tok - n_seq_decode < n_chunk)
            return fail(ATTN_E_SHAPE, "%s: %d rows cannot hold %d decode rows and %d chunks",
                        fn, n_tok, n_seq_decode, n_chunk);
        if (max_q_len <= 0 || max_q_len > n_tok - n_seq_decode)
            return fail(ATTN_E_SHAPE, "%s: max_q_len %d outside 1 .. n_tok - n_seq_decode (%d)",
                        fn, max_q_len, n_tok - n_seq_decode);
        const int g = n_head / n_head_kv;
        if (g > 128 || 128 % g != 0)
            return fail(ATTN_E_UNSUPPORTED, "%s: %d query heads per kv head (a divisor of 128)",
                        fn, g);
    } else if (n_tok != n_seq_decode) {
        return fail(ATTN_E_SHAPE, "%s: a step of decode rows only has n_tok == n_seq (%d, %d)",
                    fn, n_tok, n_seq);
    }

    // With both halves, the chunk half runs on a second stream beside the
    // decode half: the decode kernel (bound by HBM) takes seven eighths of
    // the compute units (one workgroup each), and the chunk's workgroups
    // (bound by the matrix units) start on the rest and fill in beside it.  The chunk then uses
    // four-wave workgroups, which fit on a CU next to a decode workgroup.
    // Which CU runs a row changes none of its arithmetic.
    const bool both = n_seq_decode > 0 && n_chunk > 0;
    hipEvent_t ev0 = t_ev_start, ev1 = t_ev_stop;
    t_ev_start = t_ev_stop = nullptr;
    // Decode half: sequences 0 .. n_seq_decode - 1, one row each, at token
    // rows 0 .. n_seq_decode - 1 (the step is ordered decode-first); checked
    // before anything is enqueued.
    pa::SplitArgs da;
    if (n_seq_decode > 0) {
        rc = split_setup(da, fn, 1, q, k_pool, v_pool, k_scale, v_scale, n_pages, block_table,
                         max_pages_per_seq, ctx_lens, n_seq_decode, n_head, n_head_kv, head_dim,
                         page_size, kv_dtype, out, workspace, workspace_bytes, 0, nullptr, 0, 0,
                         false);
        if (rc != ATTN_OK)
            return rc;
    }
    hipStream_t side = stream;
    hipEvent_t fork = nullptr, join = nullptr;
    if (both) {
        int cus = 0;
        rc = from_hip(side_stream(&side, &cus, &fork, &join), fn);
        if (rc != ATTN_OK)
            return rc;
        da.max_blocks = da.max_blocks > 0 ? std::min(da.max_blocks, cus * 7 / 8) : cus * 7 / 8;
    }
    if (ev0)
        (void)hipEventRecord(ev0, stream);
    if (both) {
        rc = from_hip(hipEventRecord(fork, stream), fn);
        if (rc == ATTN_OK)
            rc = from_hip(hipStreamWaitEvent(side, fork, 0), fn);
        if (rc != ATTN_OK)
            return rc;
    }
    if (n_seq_decode > 0) {
        rc = from_hip(pa::launch_split_decode(da, stream), fn);
        if (rc != ATTN_OK)
            return rc;
    }
    // Chunk half: the remaining sequences, their token rows given by the
    // absolute offsets cu_seqlens[n_seq_decode ..] into the same q and out.
    if (n_chunk > 0) {
        pa::PrefillArgs a;
        a.q = q;
        a.n_rows = 0;
        a.k_pool = k_pool;
        a.v_pool = v_pool;
        a.k_scale = k_scale;
        a.v_scale = v_scale;
        a.n_pages = n_pages;
        a.block_table = block_table + (int64_t)n_seq_decode * max_pages_per_seq;
        a.max_pages = max_pages_per_seq;
        a.ctx_len = 0;
        a.n_head = n_head;
        a.n_head_kv = n_head_kv;
        a.head_dim = head_dim;
        a.fp8 = kv_dtype == ATTN_KV_FP8_E4M3;
        a.out = out;
        a.ev_start = a.ev_stop = nullptr;
        a.cu_seqlens = cu_seqlens + n_seq_decode;
        a.ctx_lens = ctx_lens + n_seq_decode;
        a.n_var = n_chunk;
        a.max_q_len = max_q_len;
        a.n_tok = n_tok;
        a.window = 0;
        a.kv_floor = 0;
        a.narrow = both ? 1 : 0;
        rc = from_hip(pa::launch_prefill(a, side), fn);
        if (rc != ATTN_OK)
            return rc;
    }
    if (both) {
        rc = from_hip(hipEventRecord(join, side), fn);
        if (rc == ATTN_OK)
            rc = from_hip(hipStreamWaitEvent(stream, join, 0), fn);
        if (rc != ATTN_OK)
            return rc;
    }
    if (ev1)
        (void)hipEventRecord(ev1, stream);
    return ok();
}

int attn_kv_append(const void* k_new, const void* v_new, const int32_t* slot_mapping,
                   int32_t n_tok, void* k_pool, void* v_pool, float* k_scale, float* v_scale,
                   int64_t n_pages, int32_t n_head_kv, int32_t head_dim, int32_t page_size,
                   attn_kv_dtype kv_dtype, hipStream_t stream)
{
    const char* fn = "attn_kv_append";
    if (!k_new || !v_new)
        return fail(ATTN_E_ARG, "%s: k_new/v_new is NULL", fn);
    if (!slot_mapping)
        return fail(ATTN_E_ARG, "%s: slot_mapping is NULL", fn);
    if (!k_pool || !v_pool)
        return fail(ATTN_E_ARG, "%s: k_pool/v_pool is NULL", fn);
    if (kv_dtype != ATTN_KV_BF16 && kv_dtype != ATTN_KV_FP8_E4M3)
        return fail(ATTN_E_ARG, "%s: kv_dtype %d is not a kv dtype", fn, (int)kv_dtype);
    if (kv_dtype == ATTN_KV_FP8_E4M3 && (!k_scale || !v_scale))
        return fail(ATTN_E_ARG, "%s: fp8 kv needs k_scale and v_scale", fn);
    if (kv_dtype == ATTN_KV_BF16 && (k_scale || v_scale))
        return fail(ATTN_E_ARG, "%s: bf16 kv takes no scales (pass NULL)", fn);
    if (n_tok <= 0)
        return fail(ATTN_E_SHAPE, "%s: zero rows is not a call (n_tok = %d)", fn, n_tok);
    if (n_pages <= 0)
        return fail(ATTN_E_SHAPE, "%s: n_pages must be positive", fn);
    if (n_head_kv <= 0 || head_dim <= 0)
        return fail(ATTN_E_SHAPE, "%s: n_head_kv and head_dim must be positive", fn);
    if (!head_dim_ok(head_dim))
        return fail(ATTN_E_UNSUPPORTED, "%s: head_dim %d not served (128, 256)", fn, head_dim);
    if (page_size != ATTN_PAGE_SIZE)
        return fail(ATTN_E_UNSUPPORTED, "%s: page_size %d not served (16)", fn, page_size);
    if (n_head_kv > 65535)
        return fail(ATTN_E_UNSUPPORTED, "%s: n_head_kv above 65535", fn);
    pa::AppendArgs a;
    a.k_new = k_new;
    a.v_new = v_new;
    a.slots = slot_mapping;
    a.n_tok = n_tok;
    a.k_pool = k_pool;
    a.v_pool = v_pool;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    a.n_pages = n_pages;
    a.n_head_kv = n_head_kv;
    a.head_dim = head_dim;
    a.fp8 = kv_dtype == ATTN_KV_FP8_E4M3;
    return from_hip(pa::launch_append(a, stream), fn);
}

int attn_check_lengths_host(const int32_t* ctx_lens_host, int32_t n_seq, int32_t rows,
                            int32_t max_pages_per_seq, int32_t page_size)
{
    const char* fn = "attn_check_lengths_host";
    if (!ctx_lens_host)
        return fail(ATTN_E_ARG, "%s: ctx_lens_host is NULL", fn);
    if (n_seq <= 0 || rows <= 0)
        return fail(ATTN_E_SHAPE, "%s: n_seq and rows must be positive", fn);
    const int64_t cap = (int64_t)max_pages_per_seq * page_size;
    for (int32_t s = 0; s < n_seq; ++s) {
        if (ctx_lens_host[s] < rows)
            return fail(ATTN_E_RANGE, "%s: ctx_lens[%d] = %d is below the call's %d rows", fn, s,
                        ctx_lens_host[s], rows);
        if ((int64_t)ctx_lens_host[s] > cap)
            return fail(ATTN_E_RANGE, "%s: ctx_lens[%d] = %d exceeds %lld slots", fn, s,
                        ctx_lens_host[s], (long long)cap);
    }
    return ok();
}

int attn_check_block_table_host(const int32_t* block_table_host, const int32_t* ctx_lens_host,
                                int32_t n_seq, int32_t max_pages_per_seq, int32_t page_size,
                                int64_t n_pages)
{
    const char* fn = "attn_check_block_table_host";
    if (!block_table_host || !ctx_lens_host)
        return fail(ATTN_E_ARG, "%s: NULL argument", fn);
    if (n_seq <= 0 || max_pages_per_seq <= 0 || page_size <= 0)
        return fail(ATTN_E_SHAPE, "%s: sizes must be positive", fn);
    for (int32_t s = 0; s < n_seq; ++s) {
        const int64_t c = ctx_lens_host[s] < 0 ? 0 : ctx_lens_host[s];
        int64_t need = (c + page_size - 1) / page_size;
        if (need > max_pages_per_seq)
            return fail(ATTN_E_RANGE, "%s: sequence %d needs %lld pages, row holds %d", fn, s,
                        (long long)need, max_pages_per_seq);
        for (int64_t i = 0; i < need; ++i) {
            const int32_t p = block_table_host[(int64_t)s * max_pages_per_seq + i];
            if (p < 0 || (int64_t)p >= n_pages)
                return fail(ATTN_E_RANGE, "%s: block_table[%d][%lld] = %d outside [0, %lld)", fn,
                            s, (long long)i, p, (long long)n_pages);
        }
    }
    return ok();
}

}  // extern "C"
