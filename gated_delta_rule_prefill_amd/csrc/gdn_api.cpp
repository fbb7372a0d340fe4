// C ABI of libgdn.so: host-side validation, workspace sizing and launches.
// Every check happens before the first HIP call, so a rejected call launches nothing and
// touches no memory; errors are reported as status codes plus a thread-local message.
#include <hip/hip_runtime.h>

#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include <initializer_list>
#include <mutex>
#include <utility>
#include <vector>

#include "../../include/gdn.h"
#include "gdn_launch.h"

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return status;
}

int ok() {
    g_err[0] = '\0';
    return GDN_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool dim_ok(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

int check_dims(const gdn_dims_t* d) {
    if (d == nullptr) return fail(GDN_ERR_NULL, "dims is NULL");
    if (d->num_heads < 1) return fail(GDN_ERR_SHAPE, "num_heads must be >= 1 (got %d)", d->num_heads);
    if (!dim_ok(d->d_k) || !dim_ok(d->d_v))
        return fail(GDN_ERR_UNSUPPORTED, "d_k, d_v must be in {16,32,64,128} (got %d, %d)",
                    d->d_k, d->d_v);
    if (d->d_k != d->d_v)
        return fail(GDN_ERR_UNSUPPORTED, "d_k must equal d_v (got %d, %d)", d->d_k, d->d_v);
    if (d->dtype != GDN_DTYPE_F32 && d->dtype != GDN_DTYPE_BF16)
        return fail(GDN_ERR_UNSUPPORTED, "dtype must be 0 (fp32) or 1 (bf16), got %d", d->dtype);
    if (d->gate != GDN_GATE_SCALAR && d->gate != GDN_GATE_PER_KEY)
        return fail(GDN_ERR_UNSUPPORTED, "gate must be 0 (scalar) or 1 (per key), got %d", d->gate);
    if (d->qk_l2norm != 0 && d->qk_l2norm != 1)
        return fail(GDN_ERR_UNSUPPORTED, "qk_l2norm must be 0 or 1, got %d", d->qk_l2norm);
    return GDN_OK;
}

#define REQUIRE_PTR(p)                                                         \
    do {                                                                       \
        if ((p) == nullptr) return fail(GDN_ERR_NULL, "%s is NULL", #p);       \
        if (!aligned16(p)) return fail(GDN_ERR_ALIGN, "%s is not 16-byte aligned", #p); \
    } while (0)

#define OPT_PTR(p)                                                                   \
    do {                                                                             \
        if ((p) != nullptr && !aligned16(p))                                         \
            return fail(GDN_ERR_ALIGN, "%s is not 16-byte aligned", #p);             \
    } while (0)

// Debug builds (GDN_DEBUG_CHECKS) also verify what the kernels assume but the host cannot
// see without reading device memory: the valid slot indices of one call are distinct. The
// check copies the slot arrays to the host, which synchronises `stream`; release builds
// skip it. A repeated slot returns GDN_ERR_SHAPE before any launch.
#ifdef GDN_DEBUG_CHECKS
int debug_distinct_slots(std::initializer_list<std::pair<const int32_t*, int64_t>> lists,
                         int32_t n_slots, void* stream, const char* what) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    std::vector<char> seen((size_t)n_slots, 0);
    for (const auto& l : lists) {
        if (l.first == nullptr || l.second <= 0) continue;
        std::vector<int32_t> h((size_t)l.second);
        if (hipMemcpyAsync(h.data(), l.first, sizeof(int32_t) * h.size(), hipMemcpyDeviceToHost,
                           s) != hipSuccess ||
            hipStreamSynchronize(s) != hipSuccess) {
            (void)hipGetLastError();
            return fail(GDN_ERR_LAUNCH, "%s: debug check could not read the slot indices", what);
        }
        for (int32_t v : h) {
            if (v < 0 || v >= n_slots) continue;
            if (seen[(size_t)v]) return fail(GDN_ERR_SHAPE, "%s: slot %d used twice", what, v);
            seen[(size_t)v] = 1;
        }
    }
    return GDN_OK;
}
#define DEBUG_DISTINCT_SLOTS(lists, n_slots, what)                                  \
    do {                                                                            \
        int st_ = debug_distinct_slots(lists, n_slots, stream, what);               \
        if (st_) return st_;                                                        \
    } while (0)
#else
#define DEBUG_DISTINCT_SLOTS(lists, n_slots, what) \
    do {                                           \
    } while (0)
#endif
#define SLOT_LISTS(...) (std::initializer_list<std::pair<const int32_t*, int64_t>>{__VA_ARGS__})

// Workspace of the allocation-free prefill (gdn_prefill_chunked_noalloc): one copy per GPU,
// created with the library's code object on that GPU. Host code never uses the array's name
// as an address (on the host it is only a stand-in for the symbol); the device address of
// each GPU's copy comes from hipGetSymbolAddress with that GPU current, kept per device.
static __device__ __align__(256) unsigned char scratch[GDN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The current device's copy of `scratch`, resolved on the first call with that device
// current. The caller's stream must belong to that device.
int scratch_for_stream(void* stream, void** out, const char* what) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return fail(GDN_ERR_LAUNCH, "%s: no current HIP device", what);
    }
    if (dev < 0 || dev >= kMaxDevices)
        return fail(GDN_ERR_UNSUPPORTED, "%s: device %d beyond the %d the library tracks", what,
                    dev, kMaxDevices);
    if (stream != nullptr) {
        hipDevice_t sdev = -1;
        if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev) != hipSuccess) {
            (void)hipGetLastError();
            return fail(GDN_ERR_LAUNCH, "%s: cannot query the stream's device", what);
        }
        if (sdev != dev)
            return fail(GDN_ERR_UNSUPPORTED, "%s: the stream belongs to device %d, device %d is "
                                             "current", what, (int)sdev, dev);
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr) {
            (void)hipGetLastError();
            return fail(GDN_ERR_LAUNCH, "%s: hipGetSymbolAddress(scratch) failed: %s", what,
                        hipGetErrorString(e));
        }
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return GDN_OK;
}

int launch_status(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(GDN_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

int prefill_common_checks(const gdn_dims_t* dims, int32_t n_seqs, int32_t total_tokens,
                          int32_t chunk) {
    int st = check_dims(dims);
    if (st) return st;
    if (n_seqs < 0 || total_tokens < 0)
        return fail(GDN_ERR_SHAPE, "n_seqs and total_tokens must be >= 0 (got %d, %d)", n_seqs,
                    total_tokens);
    if (chunk != 16 && chunk != 32 && chunk != 64)
        return fail(GDN_ERR_UNSUPPORTED, "chunk must be 16, 32 or 64 (got %d)", chunk);
    return GDN_OK;
}

int deltalog_pool_checks(const gdn_deltalog_pool_t* pool) {
    if (pool == nullptr) return fail(GDN_ERR_NULL, "pool is NULL");
    REQUIRE_PTR(pool->base);
    REQUIRE_PTR(pool->lbar);
    REQUIRE_PTR(pool->klog);
    REQUIRE_PTR(pool->ulog);
    REQUIRE_PTR(pool->lamlog);
    REQUIRE_PTR(pool->len);
    if (pool->M < 2 || pool->M > 17)
        return fail(GDN_ERR_UNSUPPORTED, "merge interval M must be in [2, 17] (got %d)", pool->M);
    return GDN_OK;
}

// Raw projection and short-convolution operands of the conv-fused prefill.
struct ConvIn {
    const void* x;
    const float* w;
    int32_t width;
    void* state;
};

// Shared by gdn_prefill_chunked (no checkpoints), gdn_prefill_chunked_ckpt and, with conv
// set (q, k, v then unused), gdn_prefill_chunked_conv.
int prefill_run(const gdn_dims_t* dims, const void* q, const void* k, const void* v,
                const float* g, const float* beta, const int32_t* cu_seqlens, int32_t n_seqs,
                int32_t total_tokens, int32_t chunk, float* state_pool, int32_t n_slots,
                const int32_t* slots, const int32_t* has_init, const int32_t* ckpt_cu,
                const int32_t* ckpt_pos, const int32_t* ckpt_slots, int32_t n_ckpt, void* o,
                void* workspace, size_t ws_bytes, void* stream, const char* what,
                const ConvIn* conv = nullptr, bool noalloc = false) {
    int st = prefill_common_checks(dims, n_seqs, total_tokens, chunk);
    if (st) return st;
    if (conv != nullptr && (conv->width < 2 || conv->width > 4))
        return fail(GDN_ERR_UNSUPPORTED, "conv_width must be 2, 3 or 4 (got %d)", conv->width);
    if (n_seqs == 0) return ok();
    REQUIRE_PTR(cu_seqlens);
    REQUIRE_PTR(slots);
    OPT_PTR(has_init);
    REQUIRE_PTR(state_pool);
    if (n_slots < 1) return fail(GDN_ERR_SHAPE, "n_slots must be >= 1 (got %d)", n_slots);
    if (n_ckpt < 0) return fail(GDN_ERR_SHAPE, "n_ckpt must be >= 0 (got %d)", n_ckpt);
    if (n_ckpt > 0) {
        REQUIRE_PTR(ckpt_cu);
        REQUIRE_PTR(ckpt_pos);
        REQUIRE_PTR(ckpt_slots);
    }
    if (conv != nullptr) {
        const void* x = conv->x;
        const float* conv_w = conv->w;
        void* conv_state = conv->state;
        if (total_tokens > 0) REQUIRE_PTR(x);
        REQUIRE_PTR(conv_w);
        OPT_PTR(conv_state);
    }
    if (total_tokens > 0) {
        if (conv == nullptr) {
            REQUIRE_PTR(q);
            REQUIRE_PTR(k);
            REQUIRE_PTR(v);
        }
        REQUIRE_PTR(g);
        REQUIRE_PTR(beta);
        REQUIRE_PTR(o);
    }
    if (noalloc) {
        const size_t need = gdn::prefill_ws_layout(dims->dtype, dims->num_heads, dims->d_k,
                                                   dims->d_v, chunk, n_seqs, total_tokens,
                                                   nullptr, nullptr);
        if (need > GDN_NOALLOC_SCRATCH_BYTES)
            return fail(GDN_ERR_WORKSPACE, "%s: the call needs %zu bytes of workspace, the "
                                           "library's per-GPU scratch holds %zu", what, need,
                        GDN_NOALLOC_SCRATCH_BYTES);
        st = scratch_for_stream(stream, &workspace, what);
        if (st) return st;
        ws_bytes = GDN_NOALLOC_SCRATCH_BYTES;
    }
    REQUIRE_PTR(workspace);
    gdn::PrefillWs ws;
    const size_t need = gdn::prefill_ws_layout(dims->dtype, dims->num_heads, dims->d_k,
                                               dims->d_v, chunk, n_seqs, total_tokens,
                                               workspace, &ws);
    if (ws_bytes < need)
        return fail(GDN_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, need);
    gdn::PrefillArgs a;
    a.dtype = dims->dtype;
    a.gate = dims->gate;
    a.H = dims->num_heads;
    a.dk = dims->d_k;
    a.dv = dims->d_v;
    a.chunk = chunk;
    a.cp = gdn::prefill_cp(dims->dtype, chunk);
    a.l2norm = dims->qk_l2norm;
    a.scale = dims->scale;
    a.q = q;
    a.k = k;
    a.v = v;
    a.g = g;
    a.beta = beta;
    a.cu_seqlens = cu_seqlens;
    a.n_seqs = n_seqs;
    a.total_tokens = total_tokens;
    a.state_pool = state_pool;
    a.n_slots = n_slots;
    a.slots = slots;
    a.has_init = has_init;
    a.o = o;
    a.ckpt_cu = n_ckpt > 0 ? ckpt_cu : nullptr;
    a.ckpt_pos = n_ckpt > 0 ? ckpt_pos : nullptr;
    a.ckpt_slots = n_ckpt > 0 ? ckpt_slots : nullptr;
    a.n_ckpt = n_ckpt;
    a.x = conv != nullptr ? conv->x : nullptr;
    a.conv_w = conv != nullptr ? conv->w : nullptr;
    a.conv_state = conv != nullptr ? conv->state : nullptr;
    a.conv_width = conv != nullptr ? conv->width : 0;
    a.ws = ws;
    DEBUG_DISTINCT_SLOTS(SLOT_LISTS({slots, n_seqs}, {a.ckpt_slots, (int64_t)n_ckpt}), n_slots,
                         what);
    return launch_status(gdn::launch_prefill(a, static_cast<hipStream_t>(stream)), what);
}

// Shared by gdn_decode_step (spec = false: one token, num_accepted unused) and
// gdn_decode_spec (spec = true: n_pos tokens per request, num_accepted required).
int decode_run(const gdn_dims_t* dims, const void* q, const void* k, const void* v,
               const float* g, const float* beta, float* state_pool, int32_t n_slots,
               const int32_t* slots, bool spec, const int32_t* num_accepted, int32_t batch,
               int32_t n_pos, void* o, void* stream, const char* what) {
    int st = check_dims(dims);
    if (st) return st;
    if (batch < 0) return fail(GDN_ERR_SHAPE, "batch must be >= 0 (got %d)", batch);
    if (batch == 0) return ok();
    REQUIRE_PTR(q);
    REQUIRE_PTR(k);
    REQUIRE_PTR(v);
    REQUIRE_PTR(g);
    REQUIRE_PTR(beta);
    REQUIRE_PTR(state_pool);
    REQUIRE_PTR(slots);
    REQUIRE_PTR(o);
    if (spec) REQUIRE_PTR(num_accepted);
    if (n_slots < 1) return fail(GDN_ERR_SHAPE, "n_slots must be >= 1 (got %d)", n_slots);
    gdn::DecodeArgs a;
    a.dtype = dims->dtype;
    a.gate = dims->gate;
    a.H = dims->num_heads;
    a.dk = dims->d_k;
    a.dv = dims->d_v;
    a.l2norm = dims->qk_l2norm;
    a.scale = dims->scale;
    a.q = q;
    a.k = k;
    a.v = v;
    a.g = g;
    a.beta = beta;
    a.pool = state_pool;
    a.n_slots = n_slots;
    a.slots = slots;
    a.batch = batch;
    a.o = o;
    a.num_accepted = spec ? num_accepted : nullptr;
    a.n_pos = n_pos;
    DEBUG_DISTINCT_SLOTS(SLOT_LISTS({slots, (int64_t)batch * (spec ? n_pos : 1)}), n_slots, what);
    return launch_status(gdn::launch_decode(a, static_cast<hipStream_t>(stream)), what);
}

}  // namespace

extern "C" {

int gdn_prefill_workspace_bytes(const gdn_dims_t* dims, int32_t n_seqs, int32_t total_tokens,
                                int32_t chunk, size_t* bytes) {
    int st = prefill_common_checks(dims, n_seqs, total_tokens, chunk);
    if (st) return st;
    if (bytes == nullptr) return fail(GDN_ERR_NULL, "bytes is NULL");
    *bytes = gdn::prefill_ws_layout(dims->dtype, dims->num_heads, dims->d_k, dims->d_v, chunk,
                                    n_seqs, total_tokens, nullptr, nullptr);
    return ok();
}

int gdn_prefill_chunked(const gdn_dims_t* dims, const void* q, const void* k, const void* v,
                        const float* g, const float* beta, const int32_t* cu_seqlens,
                        int32_t n_seqs, int32_t total_tokens, int32_t chunk,
                        float* state_pool, int32_t n_slots, const int32_t* slots,
                        const int32_t* has_init, void* o, void* workspace, size_t ws_bytes,
                        void* stream) {
    return prefill_run(dims, q, k, v, g, beta, cu_seqlens, n_seqs, total_tokens, chunk,
                       state_pool, n_slots, slots, has_init, nullptr, nullptr, nullptr, 0, o,
                       workspace, ws_bytes, stream, "gdn_prefill_chunked");
}

int gdn_prefill_chunked_ckpt(const gdn_dims_t* dims, const void* q, const void* k,
                             const void* v, const float* g, const float* beta,
                             const int32_t* cu_seqlens, int32_t n_seqs, int32_t total_tokens,
                             int32_t chunk, float* state_pool, int32_t n_slots,
                             const int32_t* slots, const int32_t* has_init,
                             const int32_t* ckpt_cu, const int32_t* ckpt_pos,
                             const int32_t* ckpt_slots, int32_t n_ckpt, void* o,
                             void* workspace, size_t ws_bytes, void* stream) {
    return prefill_run(dims, q, k, v, g, beta, cu_seqlens, n_seqs, total_tokens, chunk,
                       state_pool, n_slots, slots, has_init, ckpt_cu, ckpt_pos, ckpt_slots,
                       n_ckpt, o, workspace, ws_bytes, stream, "gdn_prefill_chunked_ckpt");
}

int gdn_prefill_chunked_conv(const gdn_dims_t* dims, const void* x, const float* conv_w,
                             int32_t conv_width, void* conv_state, const float* g,
                             const float* beta, const int32_t* cu_seqlens, int32_t n_seqs,
                             int32_t total_tokens, int32_t chunk, float* state_pool,
                             int32_t n_slots, const int32_t* slots, const int32_t* has_init,
                             void* o, void* workspace, size_t ws_bytes, void* stream) {
    const ConvIn conv{x, conv_w, conv_width, conv_state};
    return prefill_run(dims, nullptr, nullptr, nullptr, g, beta, cu_seqlens, n_seqs,
                       total_tokens, chunk, state_pool, n_slots, slots, has_init, nullptr,
                       nullptr, nullptr, 0, o, workspace, ws_bytes, stream,
                       "gdn_prefill_chunked_conv", &conv);
}

int gdn_prefill_chunked_noalloc(const gdn_dims_t* dims, const void* q, const void* k,
                                const void* v, const float* g, const float* beta,
                                const int32_t* cu_seqlens, int32_t n_seqs,
                                int32_t total_tokens, int32_t chunk, float* state_pool,
                                int32_t n_slots, const int32_t* slots, const int32_t* has_init,
                                void* o, void* stream) {
    return prefill_run(dims, q, k, v, g, beta, cu_seqlens, n_seqs, total_tokens, chunk,
                       state_pool, n_slots, slots, has_init, nullptr, nullptr, nullptr, 0, o,
                       nullptr, 0, stream, "gdn_prefill_chunked_noalloc", nullptr, true);
}

int gdn_decode_step(const gdn_dims_t* dims, const void* q, const void* k, const void* v,
                    const float* g, const float* beta, float* state_pool, int32_t n_slots,
                    const int32_t* slots, int32_t batch, void* o, void* stream) {
    return decode_run(dims, q, k, v, g, beta, state_pool, n_slots, slots, false, nullptr, batch,
                      1, o, stream, "gdn_decode_step");
}

int gdn_decode_spec(const gdn_dims_t* dims, const void* q, const void* k, const void* v,
                    const float* g, const float* beta, float* state_pool, int32_t n_slots,
                    const int32_t* spec_slots, const int32_t* num_accepted, int32_t batch,
                    int32_t n_pos, void* o, void* stream) {
    if (n_pos < 1 || n_pos > GDN_SPEC_MAX_POS)
        return fail(GDN_ERR_UNSUPPORTED, "n_pos must be in [1, %d] (got %d)", GDN_SPEC_MAX_POS,
                    n_pos);
    return decode_run(dims, q, k, v, g, beta, state_pool, n_slots, spec_slots, true,
                      num_accepted, batch, n_pos, o, stream, "gdn_decode_spec");
}

int gdn_decode_fused(const gdn_dims_t* dims, const void* x, const float* conv_w,
                     int32_t conv_width, void* conv_state, const float* forget_b,
                     const float* write_logit, const float* A_log, const float* dt_bias,
                     float lower_bound, float* state_pool, int32_t n_slots,
                     const int32_t* slots, int32_t batch, void* o, void* stream) {
    int st = check_dims(dims);
    if (st) return st;
    if (dims->gate != GDN_GATE_PER_KEY)
        return fail(GDN_ERR_UNSUPPORTED, "the fused decode step forms per-key (KDA) gates; "
                                         "gate must be GDN_GATE_PER_KEY");
    if (conv_width < 2 || conv_width > 4)
        return fail(GDN_ERR_UNSUPPORTED, "conv_width must be 2, 3 or 4 (got %d)", conv_width);
    if (!(lower_bound < 0.f) || lower_bound < -1e30f)
        return fail(GDN_ERR_UNSUPPORTED, "lower_bound must be finite and < 0 (got %g)",
                    (double)lower_bound);
    if (batch < 0) return fail(GDN_ERR_SHAPE, "batch must be >= 0 (got %d)", batch);
    if (batch == 0) return ok();
    REQUIRE_PTR(x);
    REQUIRE_PTR(conv_w);
    REQUIRE_PTR(conv_state);
    REQUIRE_PTR(forget_b);
    REQUIRE_PTR(write_logit);
    REQUIRE_PTR(A_log);
    REQUIRE_PTR(dt_bias);
    REQUIRE_PTR(state_pool);
    REQUIRE_PTR(slots);
    REQUIRE_PTR(o);
    if (n_slots < 1) return fail(GDN_ERR_SHAPE, "n_slots must be >= 1 (got %d)", n_slots);
    gdn::FusedDecodeArgs a;
    a.dtype = dims->dtype;
    a.H = dims->num_heads;
    a.dk = dims->d_k;
    a.dv = dims->d_v;
    a.l2norm = dims->qk_l2norm;
    a.width = conv_width;
    a.scale = dims->scale;
    a.lower_bound = lower_bound;
    a.x = x;
    a.conv_w = conv_w;
    a.conv_state = conv_state;
    a.forget_b = forget_b;
    a.write_logit = write_logit;
    a.A_log = A_log;
    a.dt_bias = dt_bias;
    a.pool = state_pool;
    a.n_slots = n_slots;
    a.slots = slots;
    a.batch = batch;
    a.o = o;
    DEBUG_DISTINCT_SLOTS(SLOT_LISTS({slots, batch}), n_slots, "gdn_decode_fused");
    return launch_status(gdn::launch_fused_decode(a, static_cast<hipStream_t>(stream)),
                         "gdn_decode_fused");
}

int gdn_deltalog_workspace_bytes(const gdn_dims_t* dims, int32_t batch, int32_t M,
                                 size_t* bytes) {
    int st = check_dims(dims);
    if (st) return st;
    if (batch < 0) return fail(GDN_ERR_SHAPE, "batch must be >= 0 (got %d)", batch);
    if (M < 2 || M > 17) return fail(GDN_ERR_UNSUPPORTED, "M must be in [2, 17] (got %d)", M);
    if (bytes == nullptr) return fail(GDN_ERR_NULL, "bytes is NULL");
    *bytes = 0;
    return ok();
}

static gdn::DeltaLogArgs dl_args(const gdn_dims_t* dims, const gdn_deltalog_pool_t* pool,
                                 int32_t n_slots, const int32_t* slots, int32_t n) {
    gdn::DeltaLogArgs a = {};
    a.dtype = dims->dtype;
    a.gate = dims->gate;
    a.H = dims->num_heads;
    a.dk = dims->d_k;
    a.dv = dims->d_v;
    a.l2norm = dims->qk_l2norm;
    a.M = pool->M;
    a.scale = dims->scale;
    a.base = pool->base;
    a.lbar = pool->lbar;
    a.klog = pool->klog;
    a.ulog = pool->ulog;
    a.lamlog = pool->lamlog;
    a.len = pool->len;
    a.n_slots = n_slots;
    a.slots = slots;
    a.batch = n;
    return a;
}

int gdn_decode_deltalog(const gdn_dims_t* dims, const void* q, const void* k, const void* v,
                        const float* g, const float* beta, const gdn_deltalog_pool_t* pool,
                        int32_t n_slots, const int32_t* slots, int32_t batch, void* o,
                        void* ws, size_t ws_bytes, void* stream) {
    (void)ws;
    (void)ws_bytes;
    int st = check_dims(dims);
    if (st) return st;
    if (batch < 0) return fail(GDN_ERR_SHAPE, "batch must be >= 0 (got %d)", batch);
    st = deltalog_pool_checks(pool);
    if (st) return st;
    if (batch == 0) return ok();
    REQUIRE_PTR(q);
    REQUIRE_PTR(k);
    REQUIRE_PTR(v);
    REQUIRE_PTR(g);
    REQUIRE_PTR(beta);
    REQUIRE_PTR(slots);
    REQUIRE_PTR(o);
    if (n_slots < 1) return fail(GDN_ERR_SHAPE, "n_slots must be >= 1 (got %d)", n_slots);
    gdn::DeltaLogArgs a = dl_args(dims, pool, n_slots, slots, batch);
    a.q = q;
    a.k = k;
    a.v = v;
    a.g = g;
    a.beta = beta;
    a.o = o;
    DEBUG_DISTINCT_SLOTS(SLOT_LISTS({slots, batch}), n_slots, "gdn_decode_deltalog");
    return launch_status(gdn::launch_deltalog(a, static_cast<hipStream_t>(stream)),
                         "gdn_decode_deltalog");
}

static int deltalog_maint(const gdn_dims_t* dims, const gdn_deltalog_pool_t* pool,
                          int32_t n_slots, const int32_t* slots, int32_t n, void* stream,
                          int mode, const char* what) {
    int st = check_dims(dims);
    if (st) return st;
    st = deltalog_pool_checks(pool);
    if (st) return st;
    if (n < 0) return fail(GDN_ERR_SHAPE, "n must be >= 0 (got %d)", n);
    if (n == 0) return ok();
    REQUIRE_PTR(slots);
    if (n_slots < 1) return fail(GDN_ERR_SHAPE, "n_slots must be >= 1 (got %d)", n_slots);
    gdn::DeltaLogArgs a = dl_args(dims, pool, n_slots, slots, n);
    DEBUG_DISTINCT_SLOTS(SLOT_LISTS({slots, n}), n_slots, what);
    return launch_status(gdn::launch_deltalog_maint(a, mode, static_cast<hipStream_t>(stream)),
                         what);
}

int gdn_deltalog_reset(const gdn_dims_t* dims, const gdn_deltalog_pool_t* pool,
                       int32_t n_slots, const int32_t* slots, int32_t n, void* stream) {
    return deltalog_maint(dims, pool, n_slots, slots, n, stream, 0, "gdn_deltalog_reset");
}

int gdn_deltalog_materialize(const gdn_dims_t* dims, const gdn_deltalog_pool_t* pool,
                             int32_t n_slots, const int32_t* slots, int32_t n, void* stream) {
    return deltalog_maint(dims, pool, n_slots, slots, n, stream, 1, "gdn_deltalog_materialize");
}

int gdn_conv1d_silu(const void* x, const float* w, const int32_t* cu_seqlens, int32_t n_seqs,
                    int32_t total_tokens, int32_t channels, int32_t width, int32_t planes,
                    int32_t dtype, void* y, void* stream) {
    if (n_seqs < 0 || total_tokens < 0 || channels < 1)
        return fail(GDN_ERR_SHAPE, "bad sizes (n_seqs %d, total_tokens %d, channels %d)", n_seqs,
                    total_tokens, channels);
    if (dtype != GDN_DTYPE_F32 && dtype != GDN_DTYPE_BF16)
        return fail(GDN_ERR_UNSUPPORTED, "dtype must be 0 or 1 (got %d)", dtype);
    if (width < 2 || width > 4)
        return fail(GDN_ERR_UNSUPPORTED, "width must be 2, 3 or 4 (got %d)", width);
    if (planes < 1 || channels % (8 * planes) != 0)
        return fail(GDN_ERR_SHAPE, "channels (%d) must be a multiple of 8 * planes (%d)", channels,
                    planes);
    if (n_seqs == 0 || total_tokens == 0) return ok();
    REQUIRE_PTR(x);
    REQUIRE_PTR(w);
    REQUIRE_PTR(cu_seqlens);
    REQUIRE_PTR(y);
    gdn::ConvArgs a;
    a.dtype = dtype;
    a.channels = channels;
    a.width = width;
    a.planes = planes;
    a.n_seqs = n_seqs;
    a.total_tokens = total_tokens;
    a.x = x;
    a.w = w;
    a.cu_seqlens = cu_seqlens;
    a.y = y;
    return launch_status(gdn::launch_conv1d(a, static_cast<hipStream_t>(stream)),
                         "gdn_conv1d_silu");
}

const char* gdn_status_string(int status) {
    switch (status) {
        case GDN_OK: return "ok";
        case GDN_ERR_NULL: return "null pointer";
        case GDN_ERR_SHAPE: return "bad shape";
        case GDN_ERR_UNSUPPORTED: return "unsupported configuration";
        case GDN_ERR_ALIGN: return "misaligned pointer";
        case GDN_ERR_WORKSPACE: return "workspace too small";
        case GDN_ERR_LAUNCH: return "launch failure";
    }
    return "unknown status";
}

const char* gdn_last_error(void) { return g_err; }

int gdn_abi_version(void) { return GDN_ABI_VERSION; }

}  // extern "C"
