// lq_api.hip -- the C ABI of liblq.so: argument checks, dispatch, status.
// Every check runs before any HIP call; on an error nothing is enqueued.
#include "lq_internal.h"

#include <atomic>
#include <mutex>
#include <vector>

namespace {

thread_local int g_last_hip = 0;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Token inputs: q, k, v, o vectors 16-byte aligned; alpha 16-byte aligned in
// per-key mode and 4-byte aligned (one float per head) in scalar mode; beta
// 4-byte aligned.
int check_tokens(const lq_dims* d, const void* q, const void* k, const void* v,
                 const float* alpha, const float* beta, const void* o, bool o_required) {
    if (!q || !k || !v || !alpha || !beta || (o_required && !o)) return LQ_ERR_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || (o && !aligned16(o))) return LQ_ERR_ALIGN;
    if (d->decay_mode == LQ_DECAY_PER_KEY ? !aligned16(alpha) : !aligned4(alpha)) return LQ_ERR_ALIGN;
    if (!aligned4(beta)) return LQ_ERR_ALIGN;
    return LQ_OK;
}

int check_dims(const lq_dims* d) {
    if (!d) return LQ_ERR_NULL;
    if (d->B <= 0 || d->H <= 0 || d->dk <= 0 || d->dv <= 0 || d->W <= 0) return LQ_ERR_DIMS;
    if (d->C < 0 || d->C > d->dk) return LQ_ERR_DIMS;
    if (d->decay_mode != LQ_DECAY_SCALAR && d->decay_mode != LQ_DECAY_PER_KEY) return LQ_ERR_DIMS;
    if (d->smooth != 0 && d->smooth != 1) return LQ_ERR_DIMS;
    if (d->io_dtype != LQ_IO_F32 && d->io_dtype != LQ_IO_BF16) return LQ_ERR_DIMS;
    if ((int64_t)d->B * (int64_t)d->H > 0x7fffffffLL) return LQ_ERR_DIMS;
    if (d->dk != d->dv || (d->dk != 16 && d->dk != 64 && d->dk != 128)) return LQ_ERR_UNSUPPORTED;
    if (d->W > 32 || d->C > 8) return LQ_ERR_UNSUPPORTED;
    return LQ_OK;
}

// Codec arrays (and, if with_buffer, the window buffer) present and aligned.
int check_state(const lq_dims* d, const lq_state* st, bool with_buffer) {
    if (!st) return LQ_ERR_NULL;
    const void* req[] = {st->sq, st->row_scale, st->col_scale};
    for (const void* p : req)
        if (!p) return LQ_ERR_NULL;
    if (d->C > 0 && (!st->comp_idx || !st->comp_val)) return LQ_ERR_NULL;
    for (const void* p : req)
        if (!aligned16(p)) return LQ_ERR_ALIGN;
    if (d->C > 0 && (!aligned16(st->comp_idx) || !aligned16(st->comp_val))) return LQ_ERR_ALIGN;
    if (with_buffer) {
        const void* buf[] = {st->buf_k, st->buf_m, st->buf_g};
        for (const void* p : buf)
            if (!p) return LQ_ERR_NULL;
        for (const void* p : buf)
            if (!aligned16(p)) return LQ_ERR_ALIGN;
    }
    return LQ_OK;
}

int check_ptrs(std::initializer_list<const void*> ps) {
    for (const void* p : ps)
        if (!p) return LQ_ERR_NULL;
    for (const void* p : ps)
        if (!aligned16(p)) return LQ_ERR_ALIGN;
    return LQ_OK;
}

int finish(hipError_t e) {
    if (e != hipSuccess) {
        g_last_hip = (int)e;
        return LQ_ERR_HIP;
    }
    return LQ_OK;
}

// ---- kernel timing -----------------------------------------------------------------------------
constexpr size_t kMaxTimed = 65536;

struct TimedLaunch {
    int family;
    hipEvent_t start, stop;
};

std::mutex g_tmu;
std::atomic<bool> g_timing{false};
std::vector<TimedLaunch> g_timed;                          // this recording, in launch order
std::vector<std::pair<hipEvent_t, hipEvent_t>> g_pool;     // reused event pairs

}  // namespace

bool lq::timing_slot(int family, hipEvent_t* start, hipEvent_t* stop) {
    if (!g_timing.load(std::memory_order_relaxed)) return false;
    std::lock_guard<std::mutex> lk(g_tmu);
    if (g_timed.size() >= kMaxTimed) return false;
    if (g_timed.size() == g_pool.size()) {
        hipEvent_t a = nullptr, b = nullptr;
        if (hipEventCreate(&a) != hipSuccess) return false;
        if (hipEventCreate(&b) != hipSuccess) {
            (void)hipEventDestroy(a);
            return false;
        }
        g_pool.emplace_back(a, b);
    }
    const auto& pr = g_pool[g_timed.size()];
    g_timed.push_back({family, pr.first, pr.second});
    *start = pr.first;
    *stop = pr.second;
    return true;
}

extern "C" {

int lq_timing_enable(int32_t on) {
    std::lock_guard<std::mutex> lk(g_tmu);
    if (on) g_timed.clear();
    g_timing.store(on != 0);
    return LQ_OK;
}

int lq_timing_collect(int32_t max_records, int32_t* family, float* ms, int32_t* count) {
    if (!count || (max_records > 0 && (!family || !ms))) return LQ_ERR_NULL;
    std::lock_guard<std::mutex> lk(g_tmu);
    const int32_t n = (int32_t)g_timed.size();
    for (int32_t i = 0; i < n; ++i) {
        hipError_t e = hipEventSynchronize(g_timed[i].stop);
        if (e != hipSuccess) return finish(e);
        if (i < max_records) {
            float t = 0.0f;
            if ((e = hipEventElapsedTime(&t, g_timed[i].start, g_timed[i].stop)) != hipSuccess) return finish(e);
            family[i] = g_timed[i].family;
            ms[i] = t;
        }
    }
    g_timed.clear();
    *count = n;
    return LQ_OK;
}

}  // extern "C"

extern "C" {

int lq_check_dims(const lq_dims* d) { return check_dims(d); }

int lq_gdn_decode_step(const lq_dims* d, const lq_state* st, int32_t pos, const void* q,
                       const void* k, const void* v, const float* alpha, const float* beta,
                       void* o, void* stream) {
    int rc = check_dims(d);
    if (rc) return rc;
    if ((rc = check_state(d, st, true))) return rc;
    if ((rc = check_tokens(d, q, k, v, alpha, beta, o, true))) return rc;
    if (pos < 0) return LQ_ERR_POS;
    if (pos >= d->W) return LQ_ERR_WINDOW_FULL;
    return finish(lq::launch_decode(*d, *st, pos, nullptr, q, k, v, alpha, beta, o, (hipStream_t)stream));
}

int lq_gdn_decode_step_ragged(const lq_dims* d, const lq_state* st, const int32_t* pos,
                              const void* q, const void* k, const void* v, const float* alpha,
                              const float* beta, void* o, void* stream) {
    int rc = check_dims(d);
    if (rc) return rc;
    if ((rc = check_state(d, st, true))) return rc;
    if ((rc = check_tokens(d, q, k, v, alpha, beta, o, true))) return rc;
    if (!pos) return LQ_ERR_NULL;
    if (!aligned4(pos)) return LQ_ERR_ALIGN;
    return finish(lq::launch_decode(*d, *st, 0, pos, q, k, v, alpha, beta, o, (hipStream_t)stream));
}

int lq_gdn_window_flush(const lq_dims* d, const lq_state* st, int32_t n_buffered, float* h_out,
                        void* stream) {
    int rc = check_dims(d);
    if (rc) return rc;
    if ((rc = check_state(d, st, true))) return rc;
    if (h_out && !aligned16(h_out)) return LQ_ERR_ALIGN;
    if (n_buffered < 0 || n_buffered > d->W) return LQ_ERR_POS;
    if (n_buffered == 0) return LQ_OK;
    return finish(lq::launch_flush(*d, *st, n_buffered, nullptr, h_out, (hipStream_t)stream));
}

int lq_gdn_decode_step_flush(const lq_dims* d, const lq_state* st, int32_t pos, const void* q,
                             const void* k, const void* v, const float* alpha, const float* beta,
                             void* o, float* h_out, void* stream) {
    int rc = check_dims(d);
    if (rc) return rc;
    if ((rc = check_state(d, st, true))) return rc;
    if ((rc = check_tokens(d, q, k, v, alpha, beta, o, true))) return rc;
    if (h_out && !aligned16(h_out)) return LQ_ERR_ALIGN;
    if (pos < 0) return LQ_ERR_POS;
    if (pos >= d->W) return LQ_ERR_WINDOW_FULL;
    return finish(lq::launch_decode_flush(*d, *st, pos, nullptr, q, k, v, alpha, beta, o, h_out,
                                          (hipStream_t)stream));
}

int lq_gdn_decode_step_flush_ragged(const lq_dims* d, const lq_state* st, const int32_t* pos,
                                    const void* q, const void* k, const void* v, const float* alpha,
                                    const float* beta, void* o, float* h_out, void* stream) {
    int rc = check_dims(d);
    if (rc) return rc;
    if ((rc = check_state(d, st, true))) return rc;
    if ((rc = check_tokens(d, q, k, v, alpha, beta, o, true))) return rc;
    if (h_out && !aligned16(h_out)) return LQ_ERR_ALIGN;
    if (!pos) return LQ_ERR_NULL;
    if (!aligned4(pos)) return LQ_ERR_ALIGN;
    return finish(lq::launch_decode_flush(*d, *st, 0, pos, q, k, v, alpha, beta, o, h_out, (hipStream_t)stream));
}

int lq_gdn_window_flush_ragged(const lq_dims* d, const lq_state* st, const int32_t* n_buffered,
                               float* h_out, void* stream) {
    int rc = check_dims(d);
    if (rc) return rc;
    if ((rc = check_state(d, st, true))) return rc;
    if (h_out && !aligned16(h_out)) return LQ_ERR_ALIGN;
    if (!n_buffered) return LQ_ERR_NULL;
    if (!aligned4(n_buffered)) return LQ_ERR_ALIGN;
    return finish(lq::launch_flush(*d, *st, 0, n_buffered, h_out, (hipStream_t)stream));
}

int lq_gdn_state_quantize(const lq_dims* d, const float* h, const lq_state* st, void* stream) {
    int rc = check_dims(d);
    if (rc) return rc;
    if ((rc = check_state(d, st, false))) return rc;
    if ((rc = check_ptrs({h}))) return rc;
    return finish(lq::launch_quantize(*d, h, *st, (hipStream_t)stream));
}

int lq_gdn_state_dequantize(const lq_dims* d, const lq_state* st, float* h_out, void* stream) {
    int rc = check_dims(d);
    if (rc) return rc;
    if ((rc = check_state(d, st, false))) return rc;
    if ((rc = check_ptrs({h_out}))) return rc;
    return finish(lq::launch_dequantize(*d, *st, h_out, (hipStream_t)stream));
}

int lq_gdn_fp32_recurrence(const lq_dims* d, float* h, int32_t T, const void* q, const void* k,
                           const void* v, const float* alpha, const float* beta, void* o,
                           void* stream) {
    int rc = check_dims(d);
    if (rc) return rc;
    if ((rc = check_ptrs({h}))) return rc;
    if ((rc = check_tokens(d, q, k, v, alpha, beta, o, false))) return rc;
    if (T < 0) return LQ_ERR_POS;
    if (T == 0) return LQ_OK;
    return finish(lq::launch_fp32_recurrence(*d, h, T, q, k, v, alpha, beta, o, (hipStream_t)stream));
}

int lq_gdn_prefill(const lq_dims* d, const lq_state* st, float* h, int32_t T, const void* q,
                   const void* k, const void* v, const float* alpha, const float* beta, void* o,
                   void* stream) {
    int rc = check_dims(d);
    if (rc) return rc;
    if (st && (rc = check_state(d, st, false))) return rc;
    if ((rc = check_ptrs({h}))) return rc;
    if (T < 0) return LQ_ERR_POS;
    if (T > 0 && (rc = check_tokens(d, q, k, v, alpha, beta, o, false))) return rc;
    const hipStream_t s = (hipStream_t)stream;
    if (T > 0 && (rc = finish(lq::launch_prefill(*d, h, T, q, k, v, alpha, beta, o, s)))) return rc;
    return st ? finish(lq::launch_quantize(*d, h, *st, s)) : LQ_OK;
}

size_t lq_checkpoint_bytes(const lq_dims* d) {
    if (check_dims(d) != LQ_OK) return 0;
    return (size_t)d->B * d->H * lq::checkpoint_head_bytes(*d);
}

int lq_gdn_state_pack(const lq_dims* d, const lq_state* st, void* blob, void* stream) {
    int rc = check_dims(d);
    if (rc) return rc;
    if ((rc = check_state(d, st, false))) return rc;
    if ((rc = check_ptrs({blob}))) return rc;
    return finish(lq::launch_checkpoint(*d, *st, blob, true, (hipStream_t)stream));
}

int lq_gdn_state_unpack(const lq_dims* d, const void* blob, const lq_state* st, void* stream) {
    int rc = check_dims(d);
    if (rc) return rc;
    if ((rc = check_state(d, st, false))) return rc;
    if ((rc = check_ptrs({blob}))) return rc;
    return finish(lq::launch_checkpoint(*d, *st, const_cast<void*>(blob), false, (hipStream_t)stream));
}

size_t lq_state_bytes(const lq_dims* d) {
    if (check_dims(d) != LQ_OK) return 0;
    const size_t heads = (size_t)d->B * d->H;
    const size_t dk = d->dk, dv = d->dv, C = d->C;
    return heads * (dk * dv + 4 * dk + 4 * dv + C * (4 * dv + 4));
}

size_t lq_buffer_bytes(const lq_dims* d) {
    if (check_dims(d) != LQ_OK) return 0;
    const size_t heads = (size_t)d->B * d->H;
    const size_t gd = d->decay_mode == LQ_DECAY_PER_KEY ? d->dk : 1;
    return heads * (size_t)d->W * 4 * ((size_t)d->dk + d->dv + gd);
}

const char* lq_status_str(int status) {
    switch (status) {
        case LQ_OK: return "ok";
        case LQ_ERR_NULL: return "null pointer";
        case LQ_ERR_DIMS: return "invalid dimensions";
        case LQ_ERR_UNSUPPORTED: return "unsupported shape (dk = dv in {16, 64, 128}, W <= 32, C <= 8)";
        case LQ_ERR_WINDOW_FULL: return "window full: flush before the next decode step";
        case LQ_ERR_POS: return "window position or token count out of range";
        case LQ_ERR_ALIGN: return "misaligned pointer (16 bytes; 4 for beta and scalar alpha)";
        case LQ_ERR_HIP: return "HIP launch failed";
        default: return "unknown status";
    }
}

int lq_last_hip_error(void) { return g_last_hip; }

int lq_measure_stream_read(const void* src, size_t slice_bytes, int32_t n_slices, int32_t mode, int32_t grid,
                           void* sink, size_t write_bytes, void* stream) {
    if (!src || (write_bytes > 0 && !sink)) return LQ_ERR_NULL;
    if (!aligned16(src) || (sink && !aligned16(sink))) return LQ_ERR_ALIGN;
    if (slice_bytes < 16 || slice_bytes > 65536 || slice_bytes % 16 != 0) return LQ_ERR_DIMS;
    if (write_bytes > 4096 || write_bytes % 16 != 0) return LQ_ERR_DIMS;
    if (n_slices < 1 || (mode != 0 && mode != 1) || (mode == 1 && grid < 1)) return LQ_ERR_DIMS;
    return finish(lq::launch_stream_read(src, slice_bytes, n_slices, mode, grid, sink, write_bytes,
                                         static_cast<hipStream_t>(stream)));
}

}  // extern "C"
