// C ABI of liblbsa.so: host-side argument validation and kernel launches.
// Every check runs before anything is enqueued; the library never allocates,
// frees or synchronises.
#include <limits.h>
#include <math.h>

#include <atomic>
#include <mutex>

#include "lbsa_internal.h"

#define LBSA_API extern "C" __attribute__((visibility("default")))

using namespace lbsa;

namespace {

constexpr float kLog2eHost = 1.4426950408889634f;

int check_shape(int32_t batch, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                int32_t page_size, int32_t q_len = 1) {
    if (batch <= 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || page_size <= 0 || q_len <= 0)
        return LBSA_ERR_INVALID_ARGUMENT;
    if (q_len > kMaxQLen) return LBSA_ERR_UNSUPPORTED;
    if (num_heads % num_kv_heads != 0) return LBSA_ERR_INVALID_ARGUMENT;
    if (head_dim != kHeadDim || page_size != kTile || num_heads / num_kv_heads != kGroup)
        return LBSA_ERR_UNSUPPORTED;
    if ((long long)num_kv_heads * batch > (long long)INT_MAX / 4 ||
        (long long)num_heads * batch * q_len > (long long)INT_MAX / 4)
        return LBSA_ERR_UNSUPPORTED;
    return LBSA_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int hip_status(hipError_t e) { return e == hipSuccess ? LBSA_OK : LBSA_ERR_HIP; }

struct DecodeCommon {
    int status;
    AttnArgs a;
    bool fp8;
};

DecodeCommon check_decode(const void* q_d, const float* q_scale_d, const void* k_cache_d,
                          const void* v_cache_d, const float* k_scale_d, const float* v_scale_d,
                          int32_t kv_dtype, const int32_t* page_table_d, int32_t batch, int32_t q_len,
                          int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                          int32_t page_size, int32_t max_pages_per_seq, int64_t num_pages,
                          float softmax_scale) {
    DecodeCommon c{};
    c.status = check_shape(batch, num_heads, num_kv_heads, head_dim, page_size, q_len);
    if (c.status != LBSA_OK) return c;
    if (kv_dtype != LBSA_KV_BF16 && kv_dtype != LBSA_KV_FP8_E4M3) {
        c.status = LBSA_ERR_INVALID_ARGUMENT;
        return c;
    }
    c.fp8 = kv_dtype == LBSA_KV_FP8_E4M3;
    if (!q_d || !k_cache_d || !v_cache_d || !page_table_d || max_pages_per_seq <= 0 ||
        num_pages <= 0 || !(softmax_scale == softmax_scale)) {
        c.status = LBSA_ERR_INVALID_ARGUMENT;
        return c;
    }
    if (c.fp8 && (!q_scale_d || !k_scale_d || !v_scale_d)) {
        c.status = LBSA_ERR_INVALID_ARGUMENT;
        return c;
    }
    // 128-bit loads of K/V rows and Q, 64-bit loads of fp8 Q, 128-bit scale loads.
    if (!aligned(q_d, c.fp8 ? 8 : 16) || !aligned(k_cache_d, 16) || !aligned(v_cache_d, 16) ||
        (c.fp8 && (!aligned(k_scale_d, 16) || !aligned(v_scale_d, 16) || !aligned(q_scale_d, 4))) ||
        !aligned(page_table_d, 4)) {
        c.status = LBSA_ERR_INVALID_ARGUMENT;
        return c;
    }
    if ((long long)max_pages_per_seq * kTile > INT_MAX / 2) {
        c.status = LBSA_ERR_UNSUPPORTED;
        return c;
    }
    AttnArgs& a = c.a;
    a.q = q_d;
    a.q_scale = q_scale_d;
    a.k_cache = k_cache_d;
    a.v_cache = v_cache_d;
    a.k_scale = k_scale_d;
    a.v_scale = v_scale_d;
    a.page_table = page_table_d;
    a.num_pages = num_pages > INT32_MAX ? INT32_MAX : (int32_t)num_pages;   // every int32 page id fits
    a.B = batch;
    a.QL = q_len;
    a.Hq = num_heads;
    a.Hkv = num_kv_heads;
    a.max_pages = max_pages_per_seq;
    a.scale_log2 = softmax_scale * kLog2eHost;
    return c;
}

}  // namespace

LBSA_API const char* lbsa_status_string(int status) {
    switch (status) {
        case LBSA_OK: return "ok";
        case LBSA_ERR_INVALID_ARGUMENT: return "invalid argument";
        case LBSA_ERR_UNSUPPORTED: return "unsupported shape";
        case LBSA_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

LBSA_API int lbsa_version(void) { return 209; }

namespace {
// Events armed for the next launches on this host thread, used in order.
constexpr int kMaxArmed = 8;
thread_local hipEvent_t t_ev[kMaxArmed][2];
thread_local int t_armed = 0, t_used = 0;
thread_local unsigned long long t_launches = 0;   // launches made by this thread

void disarm() { t_armed = t_used = 0; }

// Guards a public entry point: if it returns without launching a kernel (an
// argument it rejected, or nothing to do), the timing hook is disarmed, so the
// armed events are never stamped by some later, unrelated launch.
struct HookGuard {
    unsigned long long n0 = t_launches;
    ~HookGuard() {
        if (t_launches == n0) disarm();
    }
};
}  // namespace

KernelEvents lbsa::take_kernel_events() {
    ++t_launches;
    if (t_used < t_armed) {
        const KernelEvents e{t_ev[t_used][0], t_ev[t_used][1]};
        if (++t_used == t_armed) disarm();
        return e;
    }
    return KernelEvents{nullptr, nullptr};
}

LBSA_API int lbsa_time_next_kernels(int32_t n, void* const* start_events, void* const* stop_events) {
    if (n < 0 || n > kMaxArmed || (n > 0 && (!start_events || !stop_events))) return LBSA_ERR_INVALID_ARGUMENT;
    for (int i = 0; i < n; ++i) {
        t_ev[i][0] = static_cast<hipEvent_t>(start_events[i]);
        t_ev[i][1] = static_cast<hipEvent_t>(stop_events[i]);
    }
    t_armed = n;
    t_used = 0;
    return LBSA_OK;
}

LBSA_API int lbsa_time_next_kernel(void* start_event, void* stop_event) {
    if (!start_event && !stop_event) {
        disarm();
        return LBSA_OK;
    }
    return lbsa_time_next_kernels(1, &start_event, &stop_event);
}

LBSA_API int lbsa_default_workgroups(int device, int32_t kv_dtype, int32_t q_len, int32_t* out_P) {
    if (!out_P || (kv_dtype != LBSA_KV_BF16 && kv_dtype != LBSA_KV_FP8_E4M3) || q_len < 1 || q_len > kMaxQLen)
        return LBSA_ERR_INVALID_ARGUMENT;
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess)
        return LBSA_ERR_HIP;
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) return LBSA_ERR_HIP;
    if (cur != device && hipSetDevice(device) != hipSuccess) return LBSA_ERR_HIP;
    int per_cu = 0;
    const hipError_t e = split_occupancy(kv_dtype == LBSA_KV_FP8_E4M3, q_len, &per_cu);
    if (cur != device) (void)hipSetDevice(cur);
    if (e != hipSuccess || per_cu <= 0 || cus <= 0) return LBSA_ERR_HIP;
    *out_P = cus * per_cu;
    return LBSA_OK;
}

LBSA_API int lbsa_auto_workgroups(int device, int32_t kv_dtype, int32_t q_len, int32_t num_kv_heads,
                                  int64_t total_tiles, int32_t* out_P) {
    if (!out_P || num_kv_heads <= 0 || total_tiles < 0) return LBSA_ERR_INVALID_ARGUMENT;
    int32_t resident = 0;
    const int s = lbsa_default_workgroups(device, kv_dtype, q_len, &resident);
    if (s != LBSA_OK) return s;
    // a second wave of bins when several KV heads share the batch and every
    // resident workgroup has at least kAutoTilesPerWorkgroup tiles to stream
    const bool two_waves = num_kv_heads > 1 && total_tiles >= (int64_t)kAutoTilesPerWorkgroup * resident;
    *out_P = two_waves ? 2 * resident : resident;
    return LBSA_OK;
}

LBSA_API int lbsa_task_map_layout_get(int32_t batch, int32_t num_kv_heads, int32_t P,
                                      lbsa_task_map_layout* out) {
    if (!out || batch <= 0 || num_kv_heads <= 0 || P <= 0) return LBSA_ERR_INVALID_ARGUMENT;
    const MapLayout m = map_layout(batch, num_kv_heads, P);
    out->header = m.header;
    out->bin_desc_begin = m.bin_desc_begin;
    out->desc = m.desc;
    out->seg_first_desc = m.seg_first_desc;
    out->seg_num_chunks = m.seg_num_chunks;
    out->seqlens = m.seqlens;
    out->bin_head = m.bin_head;
    out->desc_len = m.desc_len;
    out->long_seg = m.long_seg;
    out->total = m.total;
    return LBSA_OK;
}

LBSA_API int lbsa_task_map_bytes(int32_t batch, int32_t num_kv_heads, int32_t P, size_t* out_bytes) {
    if (!out_bytes) return LBSA_ERR_INVALID_ARGUMENT;
    lbsa_task_map_layout l;
    const int s = lbsa_task_map_layout_get(batch, num_kv_heads, P, &l);
    if (s == LBSA_OK) *out_bytes = l.total;
    return s;
}

LBSA_API int lbsa_workspace_layout_get(int32_t batch, int32_t q_len, int32_t num_heads,
                                       int32_t num_kv_heads, int32_t head_dim, int32_t P,
                                       lbsa_workspace_layout* out) {
    if (!out || P <= 0) return LBSA_ERR_INVALID_ARGUMENT;
    const int s = check_shape(batch, num_heads, num_kv_heads, head_dim, kTile, q_len);
    if (s != LBSA_OK) return s;
    const WsLayout w = ws_layout((size_t)num_kv_heads * batch + P, q_len);
    out->part_lse = w.part_lse;
    out->part_o = w.part_o;
    out->total = w.total;
    return LBSA_OK;
}

LBSA_API int lbsa_workspace_bytes(int32_t batch, int32_t q_len, int32_t num_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t P, size_t* out_bytes) {
    if (!out_bytes) return LBSA_ERR_INVALID_ARGUMENT;
    lbsa_workspace_layout l;
    const int s = lbsa_workspace_layout_get(batch, q_len, num_heads, num_kv_heads, head_dim, P, &l);
    if (s == LBSA_OK) *out_bytes = l.total;
    return s;
}

LBSA_API int lbsa_static_workspace_bytes(int32_t batch, int32_t q_len, int32_t num_heads,
                                         int32_t num_kv_heads, int32_t head_dim, int32_t num_splits,
                                         size_t* out_bytes) {
    if (!out_bytes || num_splits <= 0) return LBSA_ERR_INVALID_ARGUMENT;
    const int s = check_shape(batch, num_heads, num_kv_heads, head_dim, kTile, q_len);
    if (s != LBSA_OK) return s;
    *out_bytes = ws_layout((size_t)num_kv_heads * batch * num_splits, q_len).total;
    return LBSA_OK;
}

LBSA_API int lbsa_plan(const int32_t* seqlens_d, int32_t batch, int32_t num_heads,
                       int32_t num_kv_heads, int32_t page_size, int32_t max_pages_per_seq,
                       int32_t num_workgroups, int32_t min_tiles_per_bin, void* task_map_d,
                       size_t task_map_bytes, void* stream) {
    HookGuard guard;
    int s = check_shape(batch, num_heads, num_kv_heads, kHeadDim, page_size);
    if (s != LBSA_OK) return s;
    if (!seqlens_d || !task_map_d || max_pages_per_seq <= 0 || num_workgroups <= 0 ||
        min_tiles_per_bin < 0 || !aligned(task_map_d, 16) || !aligned(seqlens_d, 4))
        return LBSA_ERR_INVALID_ARGUMENT;
    // the single assign workgroup keeps (B + 1) + (Hkv*B + 1) + B ints in LDS
    if (2LL * batch + 1 + (long long)num_kv_heads * batch + 1 > kMaxAssignLdsWords)
        return LBSA_ERR_UNSUPPORTED;
    // every tile index and prefix stays far from int32 overflow
    if ((long long)batch * max_pages_per_seq * num_kv_heads >= (1LL << 30) ||
        (long long)max_pages_per_seq * kTile >= (1LL << 30) || num_workgroups >= (1 << 24))
        return LBSA_ERR_UNSUPPORTED;
    size_t need = 0;
    lbsa_task_map_bytes(batch, num_kv_heads, num_workgroups, &need);
    if (task_map_bytes < need) return LBSA_ERR_INVALID_ARGUMENT;
    const int F = min_tiles_per_bin == 0 ? LBSA_DEFAULT_MIN_TILES : min_tiles_per_bin;
    return hip_status(launch_assign(seqlens_d, batch, num_heads, num_kv_heads, num_workgroups, F,
                                    max_pages_per_seq, task_map_d,
                                    static_cast<hipStream_t>(stream)));
}

static int decode_prepare(DecodeCommon& c, int32_t batch, int32_t q_len, int32_t num_heads,
                          int32_t num_kv_heads, int32_t head_dim, int32_t num_workgroups,
                          const void* task_map_d, size_t task_map_bytes, void* workspace_d,
                          size_t workspace_bytes) {
    if (c.status != LBSA_OK) return c.status;
    if (!task_map_d || !workspace_d || num_workgroups <= 0 || !aligned(task_map_d, 16) ||
        !aligned(workspace_d, 256))
        return LBSA_ERR_INVALID_ARGUMENT;
    size_t map_need = 0, ws_need = 0;
    lbsa_task_map_bytes(batch, num_kv_heads, num_workgroups, &map_need);
    const int s = lbsa_workspace_bytes(batch, q_len, num_heads, num_kv_heads, head_dim, num_workgroups,
                                       &ws_need);
    if (s != LBSA_OK) return s;
    if (task_map_bytes < map_need || workspace_bytes < ws_need) return LBSA_ERR_INVALID_ARGUMENT;
    const WsLayout w = ws_layout((size_t)num_kv_heads * batch + num_workgroups, q_len);
    c.a.map = static_cast<const uint8_t*>(task_map_d);
    c.a.part_lse = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace_d) + w.part_lse);
    c.a.part_o = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace_d) + w.part_o);
    c.a.P = num_workgroups;
    return LBSA_OK;
}

LBSA_API int lbsa_decode_split(const void* q_d, const float* q_scale_d, const void* k_cache_d,
                               const void* v_cache_d, const float* k_scale_d, const float* v_scale_d,
                               int32_t kv_dtype, const int32_t* page_table_d, int32_t batch,
                               int32_t q_len, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                               int32_t page_size, int32_t max_pages_per_seq, int64_t num_pages,
                               int32_t num_workgroups, float softmax_scale, const void* task_map_d,
                               size_t task_map_bytes, void* workspace_d, size_t workspace_bytes,
                               void* stream) {
    HookGuard guard;
    DecodeCommon c = check_decode(q_d, q_scale_d, k_cache_d, v_cache_d, k_scale_d, v_scale_d,
                                  kv_dtype, page_table_d, batch, q_len, num_heads, num_kv_heads, head_dim,
                                  page_size, max_pages_per_seq, num_pages, softmax_scale);
    const int s = decode_prepare(c, batch, q_len, num_heads, num_kv_heads, head_dim, num_workgroups,
                                 task_map_d, task_map_bytes, workspace_d, workspace_bytes);
    if (s != LBSA_OK) return s;
    return hip_status(launch_split(c.a, c.fp8, static_cast<hipStream_t>(stream)));
}

LBSA_API int lbsa_decode_combine(int32_t batch, int32_t q_len, int32_t num_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t num_workgroups, const void* task_map_d,
                                 size_t task_map_bytes, const void* workspace_d,
                                 size_t workspace_bytes, void* out_d, void* stream) {
    HookGuard guard;
    DecodeCommon c{};
    c.status = check_shape(batch, num_heads, num_kv_heads, head_dim, kTile, q_len);
    if (c.status != LBSA_OK) return c.status;
    if (!out_d || !aligned(out_d, 8)) return LBSA_ERR_INVALID_ARGUMENT;
    c.a.B = batch;
    c.a.QL = q_len;
    c.a.Hq = num_heads;
    c.a.Hkv = num_kv_heads;
    const int s = decode_prepare(c, batch, q_len, num_heads, num_kv_heads, head_dim, num_workgroups,
                                 task_map_d, task_map_bytes, const_cast<void*>(workspace_d),
                                 workspace_bytes);
    if (s != LBSA_OK) return s;
    c.a.out = out_d;
    return hip_status(launch_combine(c.a, false, static_cast<hipStream_t>(stream)));
}

// Split + combine of lbsa_decode on prepared arguments (single-chunk segments
// written by the split kernel).
static int decode_launch(DecodeCommon& c, void* out_d, void* stream) {
    if (!out_d || !aligned(out_d, 8)) return LBSA_ERR_INVALID_ARGUMENT;
    c.a.out = out_d;
    c.a.direct_out = 1;   // single-chunk segments: the split kernel writes their rows itself
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int s = hip_status(launch_split(c.a, c.fp8, st));
    if (s != LBSA_OK) return s;
    return hip_status(launch_combine(c.a, false, st));
}

LBSA_API int lbsa_decode(const void* q_d, const float* q_scale_d, const void* k_cache_d,
                         const void* v_cache_d, const float* k_scale_d, const float* v_scale_d,
                         int32_t kv_dtype, const int32_t* page_table_d, int32_t batch, int32_t q_len,
                         int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                         int32_t page_size, int32_t max_pages_per_seq, int64_t num_pages,
                         int32_t num_workgroups, float softmax_scale, const void* task_map_d,
                         size_t task_map_bytes, void* workspace_d, size_t workspace_bytes,
                         void* out_d, void* stream) {
    HookGuard guard;
    DecodeCommon c = check_decode(q_d, q_scale_d, k_cache_d, v_cache_d, k_scale_d, v_scale_d,
                                  kv_dtype, page_table_d, batch, q_len, num_heads, num_kv_heads, head_dim,
                                  page_size, max_pages_per_seq, num_pages, softmax_scale);
    const int s = decode_prepare(c, batch, q_len, num_heads, num_kv_heads, head_dim, num_workgroups, task_map_d,
                                 task_map_bytes, workspace_d, workspace_bytes);
    if (s != LBSA_OK) return s;
    return decode_launch(c, out_d, stream);
}

// ---------------------------------------------------------------------------
// lbsa_decode without a workspace argument, for callers that cannot allocate.
// The partials live in `scratch`, a file-scope device array: every GPU the
// library runs on holds its own copy until the process ends.  In host code the
// name `scratch` is only a host-side stand-in; the kernels get the device
// address that hipGetSymbolAddress returns for the stream's device, looked up
// once per device (with that device current) and kept in scratch_ptr.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[LBSA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices];   // device address of `scratch` per device; nullptr until looked up

// Device address of `scratch` on the device that runs `stream`.
int scratch_address(hipStream_t stream, void** out) {
    int dev = -1, cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return LBSA_ERR_HIP;
    dev = cur;
    if (stream != nullptr && hipStreamGetDevice(stream, &dev) != hipSuccess) return LBSA_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return LBSA_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (scratch_ptr[dev] == nullptr) {
        if (dev != cur && hipSetDevice(dev) != hipSuccess) return LBSA_ERR_HIP;
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur) (void)hipSetDevice(cur);
        if (e != hipSuccess || p == nullptr) return LBSA_ERR_HIP;
        scratch_ptr[dev] = p;
    }
    *out = scratch_ptr[dev];
    return LBSA_OK;
}
}  // namespace

LBSA_API int lbsa_decode_noalloc(const void* q_d, const float* q_scale_d, const void* k_cache_d,
                                 const void* v_cache_d, const float* k_scale_d, const float* v_scale_d,
                                 int32_t kv_dtype, const int32_t* page_table_d, int32_t batch, int32_t q_len,
                                 int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                                 int32_t max_pages_per_seq, int64_t num_pages, int32_t num_workgroups,
                                 float softmax_scale, const void* task_map_d, size_t task_map_bytes, void* out_d,
                                 void* stream) {
    HookGuard guard;
    DecodeCommon c = check_decode(q_d, q_scale_d, k_cache_d, v_cache_d, k_scale_d, v_scale_d, kv_dtype,
                                  page_table_d, batch, q_len, num_heads, num_kv_heads, head_dim, page_size,
                                  max_pages_per_seq, num_pages, softmax_scale);
    if (c.status != LBSA_OK) return c.status;
    if (num_workgroups <= 0 || !task_map_d || !out_d) return LBSA_ERR_INVALID_ARGUMENT;
    size_t need = 0;
    int s = lbsa_workspace_bytes(batch, q_len, num_heads, num_kv_heads, head_dim, num_workgroups, &need);
    if (s != LBSA_OK) return s;
    if (need > (size_t)LBSA_NOALLOC_SCRATCH_BYTES) return LBSA_ERR_UNSUPPORTED;   // partials do not fit
    void* ws = nullptr;
    s = scratch_address(static_cast<hipStream_t>(stream), &ws);
    if (s != LBSA_OK) return s;
    s = decode_prepare(c, batch, q_len, num_heads, num_kv_heads, head_dim, num_workgroups, task_map_d,
                       task_map_bytes, ws, (size_t)LBSA_NOALLOC_SCRATCH_BYTES);
    if (s != LBSA_OK) return s;
    return decode_launch(c, out_d, stream);
}

LBSA_API int lbsa_decode_static(const void* q_d, const float* q_scale_d, const void* k_cache_d,
                                const void* v_cache_d, const float* k_scale_d,
                                const float* v_scale_d, int32_t kv_dtype,
                                const int32_t* page_table_d, const int32_t* seqlens_d,
                                int32_t batch, int32_t q_len, int32_t num_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t page_size, int32_t max_pages_per_seq,
                                int64_t num_pages, int32_t num_splits, float softmax_scale,
                                void* workspace_d, size_t workspace_bytes, void* out_d,
                                void* stream) {
    HookGuard guard;
    DecodeCommon c = check_decode(q_d, q_scale_d, k_cache_d, v_cache_d, k_scale_d, v_scale_d,
                                  kv_dtype, page_table_d, batch, q_len, num_heads, num_kv_heads, head_dim,
                                  page_size, max_pages_per_seq, num_pages, softmax_scale);
    if (c.status != LBSA_OK) return c.status;
    if (!seqlens_d || !workspace_d || !out_d || num_splits <= 0 || !aligned(workspace_d, 256) ||
        !aligned(out_d, 8) || !aligned(seqlens_d, 4))
        return LBSA_ERR_INVALID_ARGUMENT;
    if ((long long)num_splits * batch * num_kv_heads >= (1LL << 31)) return LBSA_ERR_UNSUPPORTED;
    size_t need = 0;
    const int s = lbsa_static_workspace_bytes(batch, q_len, num_heads, num_kv_heads, head_dim, num_splits,
                                              &need);
    if (s != LBSA_OK) return s;
    if (workspace_bytes < need) return LBSA_ERR_INVALID_ARGUMENT;
    const WsLayout w = ws_layout((size_t)num_kv_heads * batch * num_splits, q_len);
    c.a.seqlens = seqlens_d;
    c.a.part_lse = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace_d) + w.part_lse);
    c.a.part_o = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace_d) + w.part_o);
    c.a.out = out_d;
    c.a.P = num_splits;
    hipStream_t st = static_cast<hipStream_t>(stream);
    int r = hip_status(launch_static(c.a, c.fp8, st));
    if (r != LBSA_OK) return r;
    return hip_status(launch_combine(c.a, true, st));
}

LBSA_API int lbsa_prefill(const void* q_d, const void* k_cache_d, const void* v_cache_d, int32_t kv_dtype,
                          const int32_t* page_table_d, const int32_t* seqlens_d, int32_t batch, int32_t q_len,
                          int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                          int32_t max_pages_per_seq, int64_t num_pages, float softmax_scale, void* out_d,
                          void* stream) {
    HookGuard guard;
    const int s = check_shape(batch, num_heads, num_kv_heads, head_dim, page_size);
    if (s != LBSA_OK) return s;
    if (kv_dtype == LBSA_KV_FP8_E4M3) return LBSA_ERR_UNSUPPORTED;
    if (kv_dtype != LBSA_KV_BF16 || q_len <= 0) return LBSA_ERR_INVALID_ARGUMENT;
    if ((long long)batch * q_len * num_heads >= (1LL << 31) / kHeadDim ||
        (long long)max_pages_per_seq * kTile > INT_MAX / 2)
        return LBSA_ERR_UNSUPPORTED;
    if (!q_d || !k_cache_d || !v_cache_d || !page_table_d || !seqlens_d || !out_d || max_pages_per_seq <= 0 ||
        num_pages <= 0 || !(softmax_scale > 0.f) || !(softmax_scale < INFINITY))
        return LBSA_ERR_INVALID_ARGUMENT;
    // 16-byte Q and K/V loads, 8-byte output stores
    if (!aligned(q_d, 16) || !aligned(k_cache_d, 16) || !aligned(v_cache_d, 16) || !aligned(out_d, 8) ||
        !aligned(page_table_d, 4) || !aligned(seqlens_d, 4))
        return LBSA_ERR_INVALID_ARGUMENT;
    return hip_status(launch_prefill(q_d, k_cache_d, v_cache_d, page_table_d, seqlens_d, batch, q_len, num_heads,
                                     num_kv_heads, max_pages_per_seq, num_pages, softmax_scale * kLog2eHost, out_d,
                                     0, static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------------------
// Prefill / extend / decode rows on one task map.
// ---------------------------------------------------------------------------
static int varlen_shape(int32_t batch, int32_t num_kv_heads, int32_t P, int64_t total_q) {
    if (batch <= 0 || num_kv_heads <= 0 || P <= 0 || total_q < batch) return LBSA_ERR_INVALID_ARGUMENT;
    if (total_q > (1 << 24) || P >= (1 << 24)) return LBSA_ERR_UNSUPPORTED;
    // the single assign workgroup keeps every prefix in LDS
    if (varlen_assign_lds_words(batch, num_kv_heads, varlen_max_blocks(batch, total_q)) >
        (size_t)kMaxVarlenAssignLdsWords)
        return LBSA_ERR_UNSUPPORTED;
    return LBSA_OK;
}

static const size_t kVarlenSlotBytesLse = 4u * kVarlenRows;
static const size_t kVarlenSlotBytesO = 4u * kVarlenRows * kHeadDim;

LBSA_API int lbsa_varlen_task_map_layout_get(int32_t batch, int32_t num_kv_heads, int32_t P, int64_t total_q,
                                             lbsa_varlen_task_map_layout* out) {
    if (!out) return LBSA_ERR_INVALID_ARGUMENT;
    const int s = varlen_shape(batch, num_kv_heads, P, total_q);
    if (s != LBSA_OK) return s;
    const VarlenMapLayout m = varlen_map_layout(batch, num_kv_heads, P, varlen_max_blocks(batch, total_q));
    out->header = m.header;
    out->bin_desc_begin = m.bin_desc_begin;
    out->desc = m.desc;
    out->desc_slot = m.desc_slot;
    out->claim_order = m.claim_order;
    out->seg_first_desc = m.seg_first_desc;
    out->seg_num_chunks = m.seg_num_chunks;
    out->seg_slot0 = m.seg_slot0;
    out->blk_req = m.blk_req;
    out->blk_k = m.blk_k;
    out->qbase = m.qbase;
    out->qstart = m.qstart;
    out->seqlens = m.seqlens;
    out->qlens = m.qlens;
    out->total = m.total;
    return LBSA_OK;
}

LBSA_API int lbsa_varlen_task_map_bytes(int32_t batch, int32_t num_kv_heads, int32_t P, int64_t total_q,
                                        size_t* out_bytes) {
    if (!out_bytes) return LBSA_ERR_INVALID_ARGUMENT;
    lbsa_varlen_task_map_layout l;
    const int s = lbsa_varlen_task_map_layout_get(batch, num_kv_heads, P, total_q, &l);
    if (s == LBSA_OK) *out_bytes = l.total;
    return s;
}

LBSA_API int lbsa_varlen_workspace_bytes(int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t P,
                                         size_t* out_bytes) {
    if (!out_bytes || P <= 0) return LBSA_ERR_INVALID_ARGUMENT;
    const int s = check_shape(1, num_heads, num_kv_heads, head_dim, kTile);
    if (s != LBSA_OK) return s;
    *out_bytes = varlen_counter_bytes(P) + align_up(2 * (size_t)P * kVarlenSlotBytesLse, 256) +
                 2 * (size_t)P * kVarlenSlotBytesO;
    return LBSA_OK;
}

// Workgroups the varlen split kernel keeps resident on a device (its
// occupancy times the compute units), cached per device.
static int varlen_resident_workgroups(int device, int* out) {
    static std::atomic<int> cached[64];
    if (device >= 0 && device < 64) {
        const int c = cached[device].load(std::memory_order_relaxed);
        if (c > 0) {
            *out = c;
            return LBSA_OK;
        }
    }
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess)
        return LBSA_ERR_HIP;
    if (varlen_occupancy(&per_cu) != hipSuccess || per_cu <= 0 || cus <= 0) return LBSA_ERR_HIP;
    *out = cus * per_cu;
    if (device >= 0 && device < 64) cached[device].store(*out, std::memory_order_relaxed);
    return LBSA_OK;
}

LBSA_API int lbsa_varlen_default_workgroups(int device, int32_t* out_P) {
    if (!out_P) return LBSA_ERR_INVALID_ARGUMENT;
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess)
        return LBSA_ERR_HIP;
    if (varlen_occupancy(&per_cu) != hipSuccess || per_cu <= 0) return LBSA_ERR_HIP;
    *out_P = cus * per_cu;
    return LBSA_OK;
}

LBSA_API int lbsa_varlen_auto_workgroups(int device, const int32_t* qlens_host, int32_t batch, int32_t num_kv_heads,
                                         int32_t* out_P) {
    if (!out_P || !qlens_host || batch <= 0 || num_kv_heads <= 0) return LBSA_ERR_INVALID_ARGUMENT;
    int resident = 0;
    const int s = varlen_resident_workgroups(device, &resident);
    if (s != LBSA_OK) return s;
    int64_t nq = 0;   // query blocks; out-of-range q count none (the map marks them)
    for (int b = 0; b < batch; ++b) nq += qlens_host[b] >= 1 ? (qlens_host[b] + kQBlock - 1) / kQBlock : 0;
    // with at least 4 segments per resident workgroup the claims balance the
    // load without the extra cuts of one bin per workgroup: a quarter of the
    // bins cuts fewer segments (fewer partials and merges)
    *out_P = (int64_t)num_kv_heads * nq >= 4LL * resident ? (resident + 3) / 4 : resident;
    return LBSA_OK;
}

LBSA_API int lbsa_plan_varlen(const int32_t* seqlens_d, const int32_t* qlens_d, int32_t batch, int32_t num_heads,
                              int32_t num_kv_heads, int32_t page_size, int32_t max_pages_per_seq, int64_t total_q,
                              int32_t num_workgroups, int32_t min_tiles_per_bin, void* task_map_d,
                              size_t task_map_bytes, void* stream) {
    HookGuard guard;
    int s = check_shape(batch, num_heads, num_kv_heads, kHeadDim, page_size);
    if (s != LBSA_OK) return s;
    s = varlen_shape(batch, num_kv_heads, num_workgroups, total_q);
    if (s != LBSA_OK) return s;
    if (!seqlens_d || !qlens_d || !task_map_d || max_pages_per_seq <= 0 || min_tiles_per_bin < 0 ||
        !aligned(task_map_d, 32) || !aligned(seqlens_d, 4) || !aligned(qlens_d, 4))
        return LBSA_ERR_INVALID_ARGUMENT;
    const int64_t nq = varlen_max_blocks(batch, total_q);
    // every tile index and prefix stays far from int32 overflow
    if (nq * max_pages_per_seq * num_kv_heads >= (1LL << 30) || (long long)max_pages_per_seq * kTile >= (1LL << 30))
        return LBSA_ERR_UNSUPPORTED;
    size_t need = 0;
    lbsa_varlen_task_map_bytes(batch, num_kv_heads, num_workgroups, total_q, &need);
    if (task_map_bytes < need) return LBSA_ERR_INVALID_ARGUMENT;
    const int F = min_tiles_per_bin == 0 ? LBSA_DEFAULT_MIN_TILES : min_tiles_per_bin;
    return hip_status(launch_assign_varlen(seqlens_d, qlens_d, batch, num_heads, num_kv_heads, num_workgroups, F,
                                           max_pages_per_seq, total_q, nq, task_map_d,
                                           static_cast<hipStream_t>(stream)));
}

LBSA_API int lbsa_attend_varlen(const void* q_d, const void* k_cache_d, const void* v_cache_d,
                                const int32_t* page_table_d, int32_t batch, int32_t num_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t page_size, int32_t max_pages_per_seq, int64_t num_pages,
                                int64_t total_q, int32_t num_workgroups, float softmax_scale, const void* task_map_d,
                                size_t task_map_bytes, void* workspace_d, size_t workspace_bytes, void* out_d,
                                void* stream) {
    HookGuard guard;
    int s = check_shape(batch, num_heads, num_kv_heads, head_dim, page_size);
    if (s != LBSA_OK) return s;
    s = varlen_shape(batch, num_kv_heads, num_workgroups, total_q);
    if (s != LBSA_OK) return s;
    if (total_q * num_heads >= (1LL << 31) / kHeadDim || (long long)max_pages_per_seq * kTile > INT_MAX / 2)
        return LBSA_ERR_UNSUPPORTED;
    if (!q_d || !k_cache_d || !v_cache_d || !page_table_d || !task_map_d || !workspace_d || !out_d ||
        max_pages_per_seq <= 0 || num_pages <= 0 || !(softmax_scale > 0.f) || !(softmax_scale < INFINITY))
        return LBSA_ERR_INVALID_ARGUMENT;
    if (!aligned(q_d, 16) || !aligned(k_cache_d, 16) || !aligned(v_cache_d, 16) || !aligned(out_d, 8) ||
        !aligned(page_table_d, 4) || !aligned(task_map_d, 32) || !aligned(workspace_d, 256))
        return LBSA_ERR_INVALID_ARGUMENT;
    size_t map_need = 0, ws_need = 0;
    lbsa_varlen_task_map_bytes(batch, num_kv_heads, num_workgroups, total_q, &map_need);
    s = lbsa_varlen_workspace_bytes(num_heads, num_kv_heads, head_dim, num_workgroups, &ws_need);
    if (s != LBSA_OK) return s;
    if (task_map_bytes < map_need || workspace_bytes < ws_need) return LBSA_ERR_INVALID_ARGUMENT;
    int device = 0, resident = 0;
    if (hipGetDevice(&device) != hipSuccess) return LBSA_ERR_HIP;
    s = varlen_resident_workgroups(device, &resident);
    if (s != LBSA_OK) return s;
    // no more workgroups than the map can hold descriptors
    const int64_t nq = varlen_max_blocks(batch, total_q);
    const int64_t cap = (int64_t)num_kv_heads * nq + num_workgroups;
    const int workgroups = (int)(cap < resident ? cap : resident);
    uint8_t* ws = static_cast<uint8_t*>(workspace_d);
    int32_t* counters = reinterpret_cast<int32_t*>(ws);
    const size_t cb = varlen_counter_bytes(num_workgroups);
    float* part_lse = reinterpret_cast<float*>(ws + cb);
    float* part_o = reinterpret_cast<float*>(ws + cb + align_up(2 * (size_t)num_workgroups * kVarlenSlotBytesLse, 256));
    return hip_status(launch_varlen(q_d, k_cache_d, v_cache_d, page_table_d, task_map_d, batch, num_heads,
                                    num_kv_heads, num_workgroups, nq, max_pages_per_seq,
                                    num_pages > INT32_MAX ? INT32_MAX : num_pages, total_q,
                                    softmax_scale * kLog2eHost, counters, part_lse, part_o, out_d, workgroups,
                                    static_cast<hipStream_t>(stream)));
}

static int router_shape(int32_t m, int32_t n, int32_t k) {
    if (m < 0 || n <= 0 || k <= 0) return LBSA_ERR_INVALID_ARGUMENT;
    if (n % 16 != 0 || k % kRouterKAlign != 0 || k > (1 << 20)) return LBSA_ERR_UNSUPPORTED;
    if ((long long)m * k >= (1LL << 31) || (long long)n * k >= (1LL << 31) || (long long)m * n >= (1LL << 31))
        return LBSA_ERR_UNSUPPORTED;
    return LBSA_OK;
}

LBSA_API int lbsa_router_split_weights(const float* w_d, int32_t n, int32_t k, void* w_high_d, void* w_low_d,
                                       void* stream) {
    HookGuard guard;
    const int s = router_shape(0, n, k);
    if (s != LBSA_OK) return s;
    if (!w_d || !w_high_d || !w_low_d || !aligned(w_d, 16) || !aligned(w_high_d, 16) || !aligned(w_low_d, 16))
        return LBSA_ERR_INVALID_ARGUMENT;
    return hip_status(launch_router_split(w_d, w_high_d, w_low_d, n, k, static_cast<hipStream_t>(stream)));
}

LBSA_API int lbsa_router_workspace_bytes(int32_t m, int32_t n, int32_t k, size_t* out_bytes) {
    if (!out_bytes) return LBSA_ERR_INVALID_ARGUMENT;
    const int s = router_shape(m, n, k);
    if (s != LBSA_OK) return s;
    *out_bytes = m == 0 ? 0 : router_plan(m, n, k).workspace;
    return LBSA_OK;
}

LBSA_API int lbsa_router_gemm(const void* x_d, const void* w_high_d, const void* w_low_d, int32_t m, int32_t n,
                              int32_t k, float* scores_d, void* workspace_d, size_t workspace_bytes, void* stream) {
    HookGuard guard;
    const int s = router_shape(m, n, k);
    if (s != LBSA_OK) return s;
    if (m == 0) return LBSA_OK;
    if (!x_d || !w_high_d || !w_low_d || !scores_d || !aligned(x_d, 16) || !aligned(w_high_d, 16) ||
        !aligned(w_low_d, 16) || !aligned(scores_d, 16))
        return LBSA_ERR_INVALID_ARGUMENT;
    const RouterPlan p = router_plan(m, n, k);
    if (p.workspace > 0 && (!workspace_d || workspace_bytes < p.workspace || !aligned(workspace_d, 16)))
        return LBSA_ERR_INVALID_ARGUMENT;
    return hip_status(launch_router_gemm(x_d, w_high_d, w_low_d, m, n, k, scores_d, workspace_d,
                                         static_cast<hipStream_t>(stream)));
}

LBSA_API int lbsa_prologue(const void* qkv_d, const int32_t* positions_d, const int64_t* slot_mapping_d,
                           const float* q_norm_weight_d, const float* k_norm_weight_d, double rope_theta,
                           float eps, int32_t num_tokens, int32_t num_heads, int32_t num_kv_heads,
                           int32_t head_dim, int32_t page_size, int32_t kv_dtype, void* q_out_d,
                           float* q_scale_out_d, void* k_cache_d, void* v_cache_d, float* k_scale_d,
                           float* v_scale_d, int64_t num_pages, void* stream) {
    HookGuard guard;
    if (num_tokens < 0 || num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads != 0 ||
        num_pages <= 0)
        return LBSA_ERR_INVALID_ARGUMENT;
    if (head_dim != kHeadDim || page_size != kTile) return LBSA_ERR_UNSUPPORTED;
    if (kv_dtype != LBSA_KV_BF16 && kv_dtype != LBSA_KV_FP8_E4M3) return LBSA_ERR_INVALID_ARGUMENT;
    const bool fp8 = kv_dtype == LBSA_KV_FP8_E4M3;
    if (!(rope_theta > 1.0) || !(eps >= 0.f)) return LBSA_ERR_INVALID_ARGUMENT;
    if ((long long)num_tokens * (num_heads + 2 * num_kv_heads) >= (1LL << 31) / 4) return LBSA_ERR_UNSUPPORTED;
    if (num_tokens == 0) return LBSA_OK;
    if (!qkv_d || !positions_d || !slot_mapping_d || !q_norm_weight_d || !k_norm_weight_d || !q_out_d ||
        !k_cache_d || !v_cache_d)
        return LBSA_ERR_INVALID_ARGUMENT;
    if (fp8 && (!q_scale_out_d || !k_scale_d || !v_scale_d)) return LBSA_ERR_INVALID_ARGUMENT;
    // 16-byte loads of the projection and the weights, 16-byte bf16 / 8-byte fp8 stores
    if (!aligned(qkv_d, 16) || !aligned(positions_d, 4) || !aligned(slot_mapping_d, 8) ||
        !aligned(q_norm_weight_d, 16) || !aligned(k_norm_weight_d, 16) || !aligned(q_out_d, fp8 ? 8 : 16) ||
        !aligned(k_cache_d, fp8 ? 8 : 16) || !aligned(v_cache_d, fp8 ? 8 : 16) ||
        (fp8 && (!aligned(q_scale_out_d, 4) || !aligned(k_scale_d, 4) || !aligned(v_scale_d, 4))))
        return LBSA_ERR_INVALID_ARGUMENT;
    return hip_status(launch_prologue(static_cast<const uint16_t*>(qkv_d), positions_d, slot_mapping_d,
                                      q_norm_weight_d, k_norm_weight_d, rope_theta, eps, num_tokens,
                                      num_heads, num_kv_heads, fp8, q_out_d, q_scale_out_d, k_cache_d,
                                      v_cache_d, k_scale_d, v_scale_d, num_pages,
                                      static_cast<hipStream_t>(stream)));
}
