// qar_api.cpp -- the C ABI of libqar (declared in include/qar.h):
// synchronous argument checks, then one launch on the caller's stream.
// Nothing here allocates device memory or synchronizes.
#include "qar.h"

#include <hip/hip_runtime_api.h>

#include <stdio.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "qar_launch.h"

static_assert(QAR_MAX_RANKS == qar::kMaxRanks, "rank limit mismatch");
static_assert(QAR_CHUNK_RUN_ELEMS == qar::kChunkRunElems, "the header states the run length");
static_assert(QAR_STATIC_WORKSPACE_BYTES == qar::kStaticWorkspaceBytes, "static workspace size mismatch");

namespace {

thread_local char g_last_error[256] = "";

qar_status hip_fail(hipError_t e, const char* where) {
    snprintf(g_last_error, sizeof g_last_error, "%s: %s (%d)", where, hipGetErrorString(e), (int)e);
    return QAR_ERR_HIP;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool block_supported(uint32_t b) { return b == 64 || b == 128 || b == 256; }

size_t dtype_bytes(qar_dtype d) { return d == QAR_BF16 ? 2 : 4; }

bool dtype_ok(qar_dtype d) { return d == QAR_BF16 || d == QAR_F32; }

struct Range {
    uintptr_t lo, hi; // [lo, hi)
};

Range range(const void* p, size_t bytes) { return {(uintptr_t)p, (uintptr_t)p + bytes}; }

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

// An output may coincide exactly with an input it is allowed to replace;
// any other overlap is an error.
bool bad_overlap(Range out, Range in, bool same_allowed) {
    if (!overlap(out, in)) return false;
    return !(same_allowed && out.lo == in.lo && out.hi == in.hi);
}

// Checks common to every call: sizes, block, alignment of codes/scales.
qar_status check_common(size_t n, uint32_t block) {
    if (!block_supported(block)) return QAR_ERR_UNSUPPORTED;
    if (n % block != 0 || n > QAR_MAX_ELEMENTS) return QAR_ERR_INVALID_ARG;
    return QAR_OK;
}

// Bytes of n codes: one per element, or one per two elements for 4-bit codes.
size_t code_bytes(size_t n, int code) { return code == qar::kCodeInt4 ? n / 2 : n; }

qar_status check_reduce(const int8_t* const* codes, const float* const* scales, uint32_t nranks, size_t n,
                        uint32_t block, int8_t* codes_out, float* scales_out, void* out,
                        qar_dtype out_dtype, int code = qar::kCodeInt8) {
    qar_status st = check_common(n, block);
    if (st != QAR_OK) return st;
    if (!codes || !scales || !codes_out || !scales_out) return QAR_ERR_INVALID_ARG;
    if (nranks == 0 || nranks > QAR_MAX_RANKS) return QAR_ERR_INVALID_ARG;
    if (out && !dtype_ok(out_dtype)) return QAR_ERR_UNSUPPORTED;
    const size_t nb = n / block;
    if (!aligned(codes_out, 16) || !aligned(scales_out, 4) || (out && !aligned(out, 16)))
        return QAR_ERR_MISALIGNED;
    const size_t cb = code_bytes(n, code);
    const Range co = range(codes_out, cb), so = range(scales_out, nb * 4);
    if (overlap(co, so)) return QAR_ERR_INVALID_ARG;
    Range oo{0, 0};
    if (out) {
        oo = range(out, n * dtype_bytes(out_dtype));
        if (overlap(oo, co) || overlap(oo, so)) return QAR_ERR_INVALID_ARG;
    }
    int same_codes = -1, same_scales = -1;
    for (uint32_t r = 0; r < nranks; ++r) {
        if (!codes[r] || !scales[r]) return QAR_ERR_INVALID_ARG;
        if (!aligned(codes[r], 16) || !aligned(scales[r], 4)) return QAR_ERR_MISALIGNED;
        const Range ci = range(codes[r], cb), si = range(scales[r], nb * 4);
        if (bad_overlap(co, ci, true) || bad_overlap(so, si, true) || overlap(co, si) || overlap(so, ci))
            return QAR_ERR_INVALID_ARG;
        if (out && (overlap(oo, ci) || overlap(oo, si))) return QAR_ERR_INVALID_ARG;
        if (co.lo == ci.lo) same_codes = (int)r;
        if (so.lo == si.lo) same_scales = (int)r;
    }
    // in place means codes AND scales of the same rank
    if (same_codes != same_scales) return QAR_ERR_INVALID_ARG;
    return QAR_OK;
}

void fill_ranks(qar::RankPtrs& rp, const int8_t* const* codes, const float* const* scales, uint32_t nranks,
                size_t elem_offset, size_t block_offset) {
    memset(&rp, 0, sizeof rp);
    for (uint32_t r = 0; r < nranks; ++r) {
        rp.codes[r] = codes[r] + elem_offset;
        rp.scales[r] = scales[r] + block_offset;
    }
}

// HIP events of the calls that fork work onto side streams and join it back
// (timing disabled).  A call takes one set from its device's pool while it
// enqueues and gives it back before returning: re-recording an event does not
// disturb waits already enqueued on its previous record, so a set can serve
// the next call at once.  Sets are created on demand and kept for the life of
// the process, one per call in flight at the same time on a device (not one
// per thread).
constexpr int kEventDevices = 64;
struct EventSet {
    hipEvent_t ev[1 + QAR_MAX_STREAMS]; // ev[0]: fork, ev[1 + i]: side stream i done
};
std::mutex g_event_mu;
std::vector<EventSet*> g_event_pool[kEventDevices];

class PooledEvents {
  public:
    hipError_t acquire() {
        hipError_t e = hipGetDevice(&dev_);
        if (e != hipSuccess) return e;
        if (dev_ < 0 || dev_ >= kEventDevices) return hipErrorInvalidDevice;
        {
            std::lock_guard<std::mutex> lock(g_event_mu);
            if (!g_event_pool[dev_].empty()) {
                set_ = g_event_pool[dev_].back();
                g_event_pool[dev_].pop_back();
                return hipSuccess;
            }
        }
        EventSet* fresh = new EventSet;
        for (int i = 0; i < 1 + QAR_MAX_STREAMS; ++i) {
            e = hipEventCreateWithFlags(&fresh->ev[i], hipEventDisableTiming);
            if (e != hipSuccess) {
                for (int j = 0; j < i; ++j) (void)hipEventDestroy(fresh->ev[j]);
                delete fresh;
                return e;
            }
        }
        set_ = fresh;
        return hipSuccess;
    }
    hipEvent_t* ev() const { return set_->ev; }
    ~PooledEvents() {
        if (!set_) return;
        std::lock_guard<std::mutex> lock(g_event_mu);
        g_event_pool[dev_].push_back(set_);
    }

  private:
    int dev_ = 0;
    EventSet* set_ = nullptr;
};

// Work on streams[0 .. used-1] starts after everything already enqueued on
// `main` and `main` waits for all of it.  A side stream that is `main` itself
// needs neither, so a call whose only stream is `main` records no event.
class ForkJoin {
  public:
    ForkJoin(hipStream_t main, void* const* streams, uint32_t used) : main_(main), streams_(streams), used_(used) {
        for (uint32_t i = 0; i < used; ++i) any_side_ |= (hipStream_t)streams[i] != main;
    }
    hipError_t fork() {
        if (!any_side_) return hipSuccess;
        hipError_t e = events_.acquire();
        if (e == hipSuccess) e = hipEventRecord(events_.ev()[0], main_);
        for (uint32_t i = 0; e == hipSuccess && i < used_; ++i)
            if (is_side(i)) e = hipStreamWaitEvent(stream(i), events_.ev()[0], 0);
        return e;
    }
    hipError_t join() {
        hipError_t e = hipSuccess;
        for (uint32_t i = 0; any_side_ && e == hipSuccess && i < used_; ++i) {
            if (!is_side(i)) continue;
            e = hipEventRecord(events_.ev()[1 + i], stream(i));
            if (e == hipSuccess) e = hipStreamWaitEvent(main_, events_.ev()[1 + i], 0);
        }
        return e;
    }

  private:
    hipStream_t stream(uint32_t i) const { return (hipStream_t)streams_[i]; }
    bool is_side(uint32_t i) const { return stream(i) != main_; }
    hipStream_t main_;
    void* const* streams_;
    uint32_t used_;
    bool any_side_ = false;
    PooledEvents events_;
};

int out_kind(const void* out, qar_dtype d) {
    if (!out) return qar::kOutNone;
    return d == QAR_BF16 ? qar::kOutBF16 : qar::kOutF32;
}

} // namespace

extern "C" {

const char* qar_status_string(qar_status s) {
    switch (s) {
    case QAR_OK: return "ok";
    case QAR_ERR_INVALID_ARG: return "invalid argument";
    case QAR_ERR_MISALIGNED: return "misaligned pointer";
    case QAR_ERR_UNSUPPORTED: return "unsupported block size or dtype";
    case QAR_ERR_HIP: return "HIP runtime error";
    case QAR_ERR_CAPACITY: return "the call needs more static workspace than QAR_STATIC_WORKSPACE_BYTES";
    }
    return "unknown status";
}

const char* qar_last_error(void) { return g_last_error; }

static qar_status quantize_impl(const void* x, qar_dtype dtype, size_t n, uint32_t block, int8_t* codes,
                                float* scales, void* stream, int code, const char* name) {
    if (n == 0) return QAR_OK;
    qar_status st = check_common(n, block);
    if (st != QAR_OK) return st;
    if (!x || !codes || !scales) return QAR_ERR_INVALID_ARG;
    if (!dtype_ok(dtype)) return QAR_ERR_UNSUPPORTED;
    if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(scales, 4)) return QAR_ERR_MISALIGNED;
    const Range xi = range(x, n * dtype_bytes(dtype)), co = range(codes, code_bytes(n, code)),
                so = range(scales, n / block * 4);
    if (overlap(xi, co) || overlap(xi, so) || overlap(co, so)) return QAR_ERR_INVALID_ARG;
    const hipError_t e = qar::launch_quantize(x, dtype == QAR_BF16 ? qar::kInBF16 : qar::kInF32, n,
                                              (int)block, codes, scales, (hipStream_t)stream, code);
    return e == hipSuccess ? QAR_OK : hip_fail(e, name);
}

qar_status qar_quantize_blocks(const void* x, qar_dtype dtype, size_t n, uint32_t block, int8_t* codes,
                               float* scales, void* stream) {
    return quantize_impl(x, dtype, n, block, codes, scales, stream, qar::kCodeInt8, "qar_quantize_blocks");
}

qar_status qar_quantize_blocks_e4m3(const void* x, qar_dtype dtype, size_t n, uint32_t block, uint8_t* codes,
                                    float* scales, void* stream) {
    return quantize_impl(x, dtype, n, block, (int8_t*)codes, scales, stream, qar::kCodeE4M3,
                         "qar_quantize_blocks_e4m3");
}

qar_status qar_quantize_blocks_int4(const void* x, qar_dtype dtype, size_t n, uint32_t block, uint8_t* codes,
                                    float* scales, void* stream) {
    return quantize_impl(x, dtype, n, block, (int8_t*)codes, scales, stream, qar::kCodeInt4,
                         "qar_quantize_blocks_int4");
}

static qar_status reduce_impl(const int8_t* const* codes, const float* const* scales, uint32_t nranks, size_t n,
                              uint32_t block, int8_t* codes_out, float* scales_out, void* out, qar_dtype out_dtype,
                              void* stream, int code, const char* name) {
    if (n == 0) return QAR_OK;
    qar_status st = check_reduce(codes, scales, nranks, n, block, codes_out, scales_out, out, out_dtype, code);
    if (st != QAR_OK) return st;
    qar::RankPtrs rp;
    fill_ranks(rp, codes, scales, nranks, 0, 0);
    const hipError_t e = qar::launch_reduce(rp, (int)nranks, n, (int)block, codes_out, scales_out, out,
                                            out_kind(out, out_dtype), (hipStream_t)stream, code);
    return e == hipSuccess ? QAR_OK : hip_fail(e, name);
}

qar_status qar_reduce_quantized(const int8_t* const* codes, const float* const* scales, uint32_t nranks,
                                size_t n, uint32_t block, int8_t* codes_out, float* scales_out, void* out,
                                qar_dtype out_dtype, void* stream) {
    return reduce_impl(codes, scales, nranks, n, block, codes_out, scales_out, out, out_dtype, stream,
                       qar::kCodeInt8, "qar_reduce_quantized");
}

qar_status qar_reduce_quantized_e4m3(const uint8_t* const* codes, const float* const* scales, uint32_t nranks,
                                     size_t n, uint32_t block, uint8_t* codes_out, float* scales_out, void* out,
                                     qar_dtype out_dtype, void* stream) {
    return reduce_impl((const int8_t* const*)codes, scales, nranks, n, block, (int8_t*)codes_out, scales_out, out,
                       out_dtype, stream, qar::kCodeE4M3, "qar_reduce_quantized_e4m3");
}

qar_status qar_reduce_quantized_int4(const uint8_t* const* codes, const float* const* scales, uint32_t nranks,
                                     size_t n, uint32_t block, uint8_t* codes_out, float* scales_out, void* out,
                                     qar_dtype out_dtype, void* stream) {
    return reduce_impl((const int8_t* const*)codes, scales, nranks, n, block, (int8_t*)codes_out, scales_out, out,
                       out_dtype, stream, qar::kCodeInt4, "qar_reduce_quantized_int4");
}

static qar_status quantize_reduce_impl(const void* x_own, qar_dtype dtype, uint32_t own, int8_t* const* codes,
                                       float* const* scales, uint32_t nranks, size_t n, uint32_t block,
                                       int8_t* codes_out, float* scales_out, void* out, qar_dtype out_dtype,
                                       void* stream, int code, const char* name) {
    if (n == 0) return QAR_OK;
    if (!x_own || !codes || !scales) return QAR_ERR_INVALID_ARG;
    if (!dtype_ok(dtype)) return QAR_ERR_UNSUPPORTED;
    if (nranks == 0 || nranks > QAR_MAX_RANKS || own >= nranks) return QAR_ERR_INVALID_ARG;
    qar_status st = check_reduce((const int8_t* const*)codes, (const float* const*)scales, nranks, n, block,
                                 codes_out, scales_out, out, out_dtype, code);
    if (st != QAR_OK) return st;
    if (!aligned(x_own, 16)) return QAR_ERR_MISALIGNED;
    const size_t nb = n / block;
    // Written: rank own's codes and scales, the result (codes, scales, out).
    // Each may overlap nothing else the call reads or writes.
    const size_t cb = code_bytes(n, code);
    Range w[5] = {range(codes[own], cb), range(scales[own], nb * 4), range(codes_out, cb),
                  range(scales_out, nb * 4), out ? range(out, n * dtype_bytes(out_dtype)) : Range{0, 0}};
    const Range xi = range(x_own, n * dtype_bytes(dtype));
    for (int i = 0; i < 5; ++i)
        if (overlap(w[i], xi)) return QAR_ERR_INVALID_ARG;
    if (overlap(w[0], w[1])) return QAR_ERR_INVALID_ARG;
    for (int i = 0; i < 2; ++i) {
        for (int j = 2; j < 5; ++j)
            if (overlap(w[i], w[j])) return QAR_ERR_INVALID_ARG;
        for (uint32_t r = 0; r < nranks; ++r) {
            if (r == own) continue;
            if (overlap(w[i], range(codes[r], cb)) || overlap(w[i], range(scales[r], nb * 4)))
                return QAR_ERR_INVALID_ARG;
        }
    }
    qar::RankPtrs rp;
    fill_ranks(rp, (const int8_t* const*)codes, (const float* const*)scales, nranks, 0, 0);
    const hipError_t e = qar::launch_quantize_reduce(
        x_own, dtype == QAR_BF16 ? qar::kInBF16 : qar::kInF32, (int)own, rp, (int)nranks, n, (int)block,
        codes[own], scales[own], codes_out, scales_out, out, out_kind(out, out_dtype), (hipStream_t)stream, code);
    return e == hipSuccess ? QAR_OK : hip_fail(e, name);
}

qar_status qar_quantize_reduce(const void* x_own, qar_dtype dtype, uint32_t own, int8_t* const* codes,
                               float* const* scales, uint32_t nranks, size_t n, uint32_t block,
                               int8_t* codes_out, float* scales_out, void* out, qar_dtype out_dtype,
                               void* stream) {
    return quantize_reduce_impl(x_own, dtype, own, codes, scales, nranks, n, block, codes_out, scales_out, out,
                                out_dtype, stream, qar::kCodeInt8, "qar_quantize_reduce");
}

qar_status qar_quantize_reduce_e4m3(const void* x_own, qar_dtype dtype, uint32_t own, uint8_t* const* codes,
                                    float* const* scales, uint32_t nranks, size_t n, uint32_t block,
                                    uint8_t* codes_out, float* scales_out, void* out, qar_dtype out_dtype,
                                    void* stream) {
    return quantize_reduce_impl(x_own, dtype, own, (int8_t* const*)codes, scales, nranks, n, block,
                                (int8_t*)codes_out, scales_out, out, out_dtype, stream, qar::kCodeE4M3,
                                "qar_quantize_reduce_e4m3");
}

qar_status qar_quantize_reduce_int4(const void* x_own, qar_dtype dtype, uint32_t own, uint8_t* const* codes,
                                    float* const* scales, uint32_t nranks, size_t n, uint32_t block,
                                    uint8_t* codes_out, float* scales_out, void* out, qar_dtype out_dtype,
                                    void* stream) {
    return quantize_reduce_impl(x_own, dtype, own, (int8_t* const*)codes, scales, nranks, n, block,
                                (int8_t*)codes_out, scales_out, out, out_dtype, stream, qar::kCodeInt4,
                                "qar_quantize_reduce_int4");
}

} // extern "C"

namespace {

// The reduce as `nchunks` interleaved chunks (clipped to the number of runs
// of qar::kChunkRunElems elements): chunk c computes runs c, c + nchunks,
// ..., enqueued on streams[c % used] behind whatever that stream holds.
// Interleaved rather than contiguous chunks keep the chunks that run at
// once reading neighbouring addresses: on the small-block workload (N = 16
// × 67M, B = 64, 8 chunks over 4 streams) 200.5 -> 193.9 µs per step in a
// probe, contiguous chunks against interleaved ones in runs of 2^18
// elements, bit-identical.
hipError_t chunks_run(const int8_t* const* codes, const float* const* scales, uint32_t nranks, size_t n,
                      uint32_t block, int8_t* codes_out, float* scales_out, void* out, qar_dtype out_dtype,
                      uint32_t nchunks, void* const* streams, uint32_t used) {
    const size_t runs = qar::chunk_runs(n);
    const uint32_t chunks = (uint32_t)(nchunks < runs ? nchunks : runs);
    const int kind = out_kind(out, out_dtype);
    qar::RankPtrs rp;
    fill_ranks(rp, codes, scales, nranks, 0, 0);
    hipError_t e = hipSuccess;
    for (uint32_t c = 0; e == hipSuccess && c < chunks; ++c)
        e = qar::launch_reduce(rp, (int)nranks, n, (int)block, codes_out, scales_out, out, kind,
                               (hipStream_t)streams[c % used], qar::kCodeInt8, qar::ChunkOf{c, chunks});
    return e;
}

uint32_t streams_used(uint32_t nchunks, size_t n, uint32_t nstreams) {
    const size_t runs = qar::chunk_runs(n);
    const size_t chunks = nchunks < runs ? nchunks : runs;
    return (uint32_t)(chunks < nstreams ? chunks : nstreams);
}

} // namespace

extern "C" {

qar_status qar_reduce_quantized_chunked(const int8_t* const* codes, const float* const* scales, uint32_t nranks,
                                        size_t n, uint32_t block, int8_t* codes_out, float* scales_out, void* out,
                                        qar_dtype out_dtype, uint32_t nchunks, void* const* streams,
                                        uint32_t nstreams) {
    if (n == 0) return QAR_OK;
    qar_status st = check_reduce(codes, scales, nranks, n, block, codes_out, scales_out, out, out_dtype);
    if (st != QAR_OK) return st;
    if (nchunks == 0 || !streams || nstreams == 0 || nstreams > QAR_MAX_STREAMS) return QAR_ERR_INVALID_ARG;
    const hipError_t e = chunks_run(codes, scales, nranks, n, block, codes_out, scales_out, out, out_dtype, nchunks,
                                    streams, streams_used(nchunks, n, nstreams));
    return e == hipSuccess ? QAR_OK : hip_fail(e, "qar_reduce_quantized_chunked");
}

qar_status qar_reduce_quantized_pipelined(const int8_t* const* codes, const float* const* scales,
                                          uint32_t nranks, size_t n, uint32_t block, int8_t* codes_out,
                                          float* scales_out, void* out, qar_dtype out_dtype,
                                          uint32_t nchunks, void* const* streams, uint32_t nstreams,
                                          void* stream) {
    if (n == 0) return QAR_OK;
    qar_status st = check_reduce(codes, scales, nranks, n, block, codes_out, scales_out, out, out_dtype);
    if (st != QAR_OK) return st;
    if (nchunks == 0 || !streams || nstreams == 0 || nstreams > QAR_MAX_STREAMS) return QAR_ERR_INVALID_ARG;
    // NULL (the default stream) only as the calling stream itself
    for (uint32_t i = 0; i < nstreams; ++i)
        if (!streams[i] && stream) return QAR_ERR_INVALID_ARG;
    const uint32_t used = streams_used(nchunks, n, nstreams);
    ForkJoin fj((hipStream_t)stream, streams, used);
    hipError_t e = fj.fork();
    if (e == hipSuccess)
        e = chunks_run(codes, scales, nranks, n, block, codes_out, scales_out, out, out_dtype, nchunks, streams, used);
    if (e == hipSuccess) e = fj.join();
    return e == hipSuccess ? QAR_OK : hip_fail(e, "qar_reduce_quantized_pipelined");
}

static qar_status ring_step_impl(const int8_t* codes_in, const float* scales_in, const void* local,
                                 qar_dtype dtype, size_t n, uint32_t block, int8_t* codes_out, float* scales_out,
                                 void* stream, int code, const char* name) {
    if (n == 0) return QAR_OK;
    qar_status st = check_common(n, block);
    if (st != QAR_OK) return st;
    if (!codes_in || !scales_in || !local || !codes_out || !scales_out) return QAR_ERR_INVALID_ARG;
    if (!dtype_ok(dtype)) return QAR_ERR_UNSUPPORTED;
    if (!aligned(codes_in, 16) || !aligned(codes_out, 16) || !aligned(local, 16) || !aligned(scales_in, 4) ||
        !aligned(scales_out, 4))
        return QAR_ERR_MISALIGNED;
    const size_t nb = n / block;
    const size_t cb = code_bytes(n, code);
    const Range ci = range(codes_in, cb), si = range(scales_in, nb * 4), li = range(local, n * dtype_bytes(dtype)),
                co = range(codes_out, cb), so = range(scales_out, nb * 4);
    if (bad_overlap(co, ci, true) || bad_overlap(so, si, true) || overlap(co, si) || overlap(so, ci) ||
        overlap(co, li) || overlap(so, li) || overlap(co, so))
        return QAR_ERR_INVALID_ARG;
    if ((co.lo == ci.lo) != (so.lo == si.lo)) return QAR_ERR_INVALID_ARG;
    const hipError_t e =
        qar::launch_ring_step(codes_in, scales_in, local, dtype == QAR_BF16 ? qar::kInBF16 : qar::kInF32, n,
                              (int)block, codes_out, scales_out, (hipStream_t)stream, code);
    return e == hipSuccess ? QAR_OK : hip_fail(e, name);
}

qar_status qar_ring_step(const int8_t* codes_in, const float* scales_in, const void* local, qar_dtype dtype,
                         size_t n, uint32_t block, int8_t* codes_out, float* scales_out, void* stream) {
    return ring_step_impl(codes_in, scales_in, local, dtype, n, block, codes_out, scales_out, stream,
                          qar::kCodeInt8, "qar_ring_step");
}

qar_status qar_ring_step_e4m3(const uint8_t* codes_in, const float* scales_in, const void* local,
                              qar_dtype dtype, size_t n, uint32_t block, uint8_t* codes_out, float* scales_out,
                              void* stream) {
    return ring_step_impl((const int8_t*)codes_in, scales_in, local, dtype, n, block, (int8_t*)codes_out,
                          scales_out, stream, qar::kCodeE4M3, "qar_ring_step_e4m3");
}

qar_status qar_ring_step_int4(const uint8_t* codes_in, const float* scales_in, const void* local,
                              qar_dtype dtype, size_t n, uint32_t block, uint8_t* codes_out, float* scales_out,
                              void* stream) {
    return ring_step_impl((const int8_t*)codes_in, scales_in, local, dtype, n, block, (int8_t*)codes_out,
                          scales_out, stream, qar::kCodeInt4, "qar_ring_step_int4");
}

static qar_status dequantize_impl(const int8_t* codes, const float* scales, size_t n, uint32_t block, void* out,
                                  qar_dtype out_dtype, void* stream, int code, const char* name) {
    if (n == 0) return QAR_OK;
    qar_status st = check_common(n, block);
    if (st != QAR_OK) return st;
    if (!codes || !scales || !out) return QAR_ERR_INVALID_ARG;
    if (!dtype_ok(out_dtype)) return QAR_ERR_UNSUPPORTED;
    if (!aligned(codes, 16) || !aligned(scales, 4) || !aligned(out, 16)) return QAR_ERR_MISALIGNED;
    const Range ci = range(codes, code_bytes(n, code)), si = range(scales, n / block * 4),
                oo = range(out, n * dtype_bytes(out_dtype));
    if (overlap(oo, ci) || overlap(oo, si)) return QAR_ERR_INVALID_ARG;
    const hipError_t e = qar::launch_dequantize(codes, scales, n, (int)block, out, out_kind(out, out_dtype),
                                                (hipStream_t)stream, code);
    return e == hipSuccess ? QAR_OK : hip_fail(e, name);
}

qar_status qar_dequantize(const int8_t* codes, const float* scales, size_t n, uint32_t block, void* out,
                          qar_dtype out_dtype, void* stream) {
    return dequantize_impl(codes, scales, n, block, out, out_dtype, stream, qar::kCodeInt8, "qar_dequantize");
}

qar_status qar_dequantize_e4m3(const uint8_t* codes, const float* scales, size_t n, uint32_t block, void* out,
                               qar_dtype out_dtype, void* stream) {
    return dequantize_impl((const int8_t*)codes, scales, n, block, out, out_dtype, stream, qar::kCodeE4M3,
                           "qar_dequantize_e4m3");
}

qar_status qar_dequantize_int4(const uint8_t* codes, const float* scales, size_t n, uint32_t block, void* out,
                               qar_dtype out_dtype, void* stream) {
    return dequantize_impl((const int8_t*)codes, scales, n, block, out, out_dtype, stream, qar::kCodeInt4,
                           "qar_dequantize_int4");
}

qar_status qar_reduce_unquantized(const void* const* x, uint32_t nranks, size_t n, qar_dtype dtype, void* out,
                                  void* stream) {
    if (n == 0) return QAR_OK;
    if (!x || !out || nranks == 0 || nranks > QAR_MAX_RANKS) return QAR_ERR_INVALID_ARG;
    if (!dtype_ok(dtype)) return QAR_ERR_UNSUPPORTED;
    if (n % 16 != 0 || n > QAR_MAX_ELEMENTS) return QAR_ERR_INVALID_ARG;
    if (!aligned(out, 16)) return QAR_ERR_MISALIGNED;
    const size_t bytes = n * dtype_bytes(dtype);
    const Range oo = range(out, bytes);
    qar::PlainPtrs xp;
    memset(&xp, 0, sizeof xp);
    for (uint32_t r = 0; r < nranks; ++r) {
        if (!x[r]) return QAR_ERR_INVALID_ARG;
        if (!aligned(x[r], 16)) return QAR_ERR_MISALIGNED;
        if (bad_overlap(oo, range(x[r], bytes), true)) return QAR_ERR_INVALID_ARG;
        xp.x[r] = x[r];
    }
    const hipError_t e = qar::launch_reduce_unquantized(xp, (int)nranks, n, dtype == QAR_BF16 ? qar::kInBF16 : qar::kInF32,
                                                        out, (hipStream_t)stream);
    return e == hipSuccess ? QAR_OK : hip_fail(e, "qar_reduce_unquantized");
}

} // extern "C"

namespace {

// Checks shared by both simulated-AllReduce calls: sizes, inputs, output.
qar_status check_allreduce(const void* const* x, qar_dtype dtype, uint32_t nranks, size_t n, uint32_t block,
                           qar_schedule schedule, void* out, uint32_t nchunks, Range* ins, Range* oo) {
    qar_status st = check_common(n, block);
    if (st != QAR_OK) return st;
    if (schedule != QAR_SCHEDULE_ONE_SHOT && schedule != QAR_SCHEDULE_RING) return QAR_ERR_UNSUPPORTED;
    if (!dtype_ok(dtype)) return QAR_ERR_UNSUPPORTED;
    if (!x || !out) return QAR_ERR_INVALID_ARG;
    if (nranks == 0 || nranks > QAR_MAX_RANKS || nchunks == 0) return QAR_ERR_INVALID_ARG;
    const size_t eb = dtype_bytes(dtype);
    for (uint32_t r = 0; r < nranks; ++r) {
        if (!x[r]) return QAR_ERR_INVALID_ARG;
        if (!aligned(x[r], 16)) return QAR_ERR_MISALIGNED;
        ins[r] = range(x[r], n * eb);
    }
    if (!aligned(out, 16)) return QAR_ERR_MISALIGNED;
    *oo = range(out, n * eb);
    for (uint32_t r = 0; r < nranks; ++r)
        if (overlap(*oo, ins[r])) return QAR_ERR_INVALID_ARG;
    return QAR_OK;
}

// The simulated AllReduce after its checks: chunk c on streams[c % used],
// staging in codes_work / scales_work (nranks of each for one-shot, [0] for
// the ring).
hipError_t allreduce_run(const void* const* x, qar_dtype dtype, uint32_t nranks, size_t n, uint32_t block,
                         qar_schedule schedule, int8_t* const* codes_work, float* const* scales_work, void* out,
                         uint32_t nchunks, void* const* streams, uint32_t nstreams, hipStream_t main_st) {
    const size_t nb = n / block, eb = dtype_bytes(dtype);
    const size_t chunks = nchunks < nb ? nchunks : nb;
    const size_t per = (nb + chunks - 1) / chunks;
    const uint32_t used = (uint32_t)(chunks < nstreams ? chunks : nstreams);
    const int kind = dtype == QAR_BF16 ? qar::kInBF16 : qar::kInF32;
    const int okind = dtype == QAR_BF16 ? qar::kOutBF16 : qar::kOutF32;

    ForkJoin fj(main_st, streams, used);
    hipError_t e = fj.fork();
    for (size_t c = 0; e == hipSuccess && c < chunks; ++c) {
        const size_t b0 = c * per;
        if (b0 >= nb) break;
        const size_t bn = (nb - b0 < per) ? nb - b0 : per, e0 = b0 * block, cn = bn * block;
        const hipStream_t cs = (hipStream_t)streams[c % used];
        const auto xin = [&](uint32_t r) { return (const void*)((const char*)x[r] + e0 * eb); };
        void* const oc = (void*)((char*)out + e0 * eb);
        if (schedule == QAR_SCHEDULE_ONE_SHOT) {
            // ranks 0..N-2 quantized on their own; the last rank's quantize
            // runs inside the reduce (one launch and one re-read fewer); the
            // result replaces rank 0's codes, which each lane reads first
            qar::RankPtrs rp;
            memset(&rp, 0, sizeof rp);
            const uint32_t last = nranks - 1;
            for (uint32_t r = 0; r < nranks; ++r) {
                rp.codes[r] = codes_work[r] + e0;
                rp.scales[r] = scales_work[r] + b0;
            }
            for (uint32_t r = 0; e == hipSuccess && r < (nranks > 1 ? last : nranks); ++r)
                e = qar::launch_quantize(xin(r), kind, cn, (int)block, codes_work[r] + e0, scales_work[r] + b0, cs);
            if (e == hipSuccess && nranks > 1)
                e = qar::launch_quantize_reduce(xin(last), kind, (int)last, rp, (int)nranks, cn, (int)block,
                                                codes_work[last] + e0, scales_work[last] + b0, codes_work[0] + e0,
                                                scales_work[0] + b0, oc, okind, cs);
            else if (e == hipSuccess)
                e = qar::launch_reduce(rp, 1, cn, (int)block, codes_work[0] + e0, scales_work[0] + b0, oc, okind, cs);
        } else {
            const uint32_t s0 = (uint32_t)(c % nranks);
            int8_t* const q = codes_work[0] + e0;
            float* const sc = scales_work[0] + b0;
            e = qar::launch_quantize(xin(s0), kind, cn, (int)block, q, sc, cs);
            for (uint32_t k = 1; e == hipSuccess && k < nranks; ++k)
                e = qar::launch_ring_step(q, sc, xin((s0 + k) % nranks), kind, cn, (int)block, q, sc, cs);
            if (e == hipSuccess) e = qar::launch_dequantize(q, sc, cn, (int)block, oc, okind, cs);
        }
    }
    if (e == hipSuccess) e = fj.join();
    return e;
}

// Byte offsets of the staging inside the static workspace: rank r's codes at
// r * code_stride, its scales at nwork * code_stride + r * scale_stride; both
// strides are multiples of 256 bytes.
struct StaticLayout {
    size_t code_stride, scale_stride, bytes;
};

StaticLayout static_layout(uint32_t nwork, size_t n, size_t nb) {
    StaticLayout l;
    l.code_stride = (n + 255) / 256 * 256;
    l.scale_stride = (nb * 4 + 255) / 256 * 256;
    l.bytes = nwork * (l.code_stride + l.scale_stride);
    return l;
}

} // namespace

extern "C" {

qar_status qar_allreduce_simulated(const void* const* x, qar_dtype dtype, uint32_t nranks, size_t n,
                                   uint32_t block, qar_schedule schedule, int8_t* const* codes_work,
                                   float* const* scales_work, void* out, uint32_t nchunks,
                                   void* const* streams, uint32_t nstreams, void* stream) {
    if (n == 0) return QAR_OK;
    Range ins[QAR_MAX_RANKS], oo;
    qar_status st = check_allreduce(x, dtype, nranks, n, block, schedule, out, nchunks, ins, &oo);
    if (st != QAR_OK) return st;
    if (!codes_work || !scales_work || !streams) return QAR_ERR_INVALID_ARG;
    if (nstreams == 0 || nstreams > QAR_MAX_STREAMS) return QAR_ERR_INVALID_ARG;
    for (uint32_t i = 0; i < nstreams; ++i)
        if (!streams[i] && stream) return QAR_ERR_INVALID_ARG;
    const uint32_t nwork = schedule == QAR_SCHEDULE_ONE_SHOT ? nranks : 1;
    const size_t nb = n / block;
    // the workspaces and the output may overlap nothing; inputs may overlap
    // each other
    Range outs[2 * QAR_MAX_RANKS + 1];
    int nouts = 0;
    for (uint32_t r = 0; r < nwork; ++r) {
        if (!codes_work[r] || !scales_work[r]) return QAR_ERR_INVALID_ARG;
        if (!aligned(codes_work[r], 16) || !aligned(scales_work[r], 4)) return QAR_ERR_MISALIGNED;
        outs[nouts++] = range(codes_work[r], n);
        outs[nouts++] = range(scales_work[r], nb * 4);
    }
    outs[nouts++] = oo;
    for (int i = 0; i < nouts; ++i) {
        for (int j = i + 1; j < nouts; ++j)
            if (overlap(outs[i], outs[j])) return QAR_ERR_INVALID_ARG;
        for (uint32_t r = 0; r < nranks; ++r)
            if (overlap(outs[i], ins[r])) return QAR_ERR_INVALID_ARG;
    }
    const hipError_t e = allreduce_run(x, dtype, nranks, n, block, schedule, codes_work, scales_work, out, nchunks,
                                       streams, nstreams, (hipStream_t)stream);
    return e == hipSuccess ? QAR_OK : hip_fail(e, "qar_allreduce_simulated");
}

qar_status qar_allreduce_simulated_static(const void* const* x, qar_dtype dtype, uint32_t nranks, size_t n,
                                          uint32_t block, qar_schedule schedule, void* out, uint32_t nchunks,
                                          void* stream) {
    if (n == 0) return QAR_OK;
    Range ins[QAR_MAX_RANKS], oo;
    qar_status st = check_allreduce(x, dtype, nranks, n, block, schedule, out, nchunks, ins, &oo);
    if (st != QAR_OK) return st;
    const uint32_t nwork = schedule == QAR_SCHEDULE_ONE_SHOT ? nranks : 1;
    const size_t nb = n / block;
    const StaticLayout l = static_layout(nwork, n, nb);
    if (l.bytes > QAR_STATIC_WORKSPACE_BYTES) {
        snprintf(g_last_error, sizeof g_last_error,
                 "qar_allreduce_simulated_static: needs %zu bytes of static workspace, the limit is %zu", l.bytes,
                 (size_t)QAR_STATIC_WORKSPACE_BYTES);
        return QAR_ERR_CAPACITY;
    }
    uint8_t* base = nullptr;
    const hipError_t ew = qar::static_workspace(&base);
    if (ew != hipSuccess) return hip_fail(ew, "qar_allreduce_simulated_static: workspace address");
    int8_t* codes_work[QAR_MAX_RANKS];
    float* scales_work[QAR_MAX_RANKS];
    for (uint32_t r = 0; r < nwork; ++r) {
        codes_work[r] = reinterpret_cast<int8_t*>(base + r * l.code_stride);
        scales_work[r] = reinterpret_cast<float*>(base + nwork * l.code_stride + r * l.scale_stride);
    }
    void* const streams[1] = {stream};
    const hipError_t e = allreduce_run(x, dtype, nranks, n, block, schedule, codes_work, scales_work, out, nchunks,
                                       streams, 1, (hipStream_t)stream);
    return e == hipSuccess ? QAR_OK : hip_fail(e, "qar_allreduce_simulated_static");
}

} // extern "C"

// ---------------------------------------------------------------------------
// row-bounded blocks

namespace {

struct RowShape {
    size_t rows, row_len, per_row, nblocks, n;
};

qar_status row_shape(size_t rows, size_t row_len, uint32_t block, RowShape& sh) {
    if (!block_supported(block)) return QAR_ERR_UNSUPPORTED;
    if (row_len != 0 && rows > QAR_MAX_ELEMENTS / row_len) return QAR_ERR_INVALID_ARG;
    sh.rows = rows;
    sh.row_len = row_len;
    sh.per_row = (row_len + block - 1) / block;
    sh.n = rows * row_len;
    sh.nblocks = rows * sh.per_row;
    if (sh.nblocks > QAR_MAX_ROW_BLOCKS) return QAR_ERR_INVALID_ARG;
    return QAR_OK;
}

bool flat_ok(const RowShape& sh, uint32_t block) { return sh.row_len % block == 0; }

qar::RowsCall rows_call(int op, const RowShape& sh, uint32_t block) {
    qar::RowsCall c;
    memset(&c, 0, sizeof c);
    c.op = op;
    c.rows = sh.rows;
    c.row_len = sh.row_len;
    c.block = (int)block;
    return c;
}

} // namespace

extern "C" {

qar_status qar_quantize_rows(const void* x, qar_dtype dtype, size_t rows, size_t row_len, uint32_t block,
                             int8_t* codes, float* scales, void* stream) {
    RowShape sh;
    qar_status st = row_shape(rows, row_len, block, sh);
    if (st != QAR_OK || sh.n == 0) return st;
    if (!x || !codes || !scales) return QAR_ERR_INVALID_ARG;
    if (!dtype_ok(dtype)) return QAR_ERR_UNSUPPORTED;
    if (flat_ok(sh, block) && aligned(x, 16) && aligned(codes, 16))
        return qar_quantize_blocks(x, dtype, sh.n, block, codes, scales, stream);
    if (!aligned(x, dtype_bytes(dtype)) || !aligned(scales, 4)) return QAR_ERR_MISALIGNED;
    const Range xi = range(x, sh.n * dtype_bytes(dtype)), co = range(codes, sh.n), so = range(scales, sh.nblocks * 4);
    if (overlap(xi, co) || overlap(xi, so) || overlap(co, so)) return QAR_ERR_INVALID_ARG;
    qar::RowsCall c = rows_call(qar::kRowsQuantize, sh, block);
    c.vector = sh.row_len % 16 == 0 && aligned(x, 16) && aligned(codes, 16);
    c.kind = dtype == QAR_BF16 ? qar::kInBF16 : qar::kInF32;
    c.x = x;
    c.codes_out = codes;
    c.scales_out = scales;
    const hipError_t e = qar::launch_rows(c, (hipStream_t)stream);
    return e == hipSuccess ? QAR_OK : hip_fail(e, "qar_quantize_rows");
}

qar_status qar_dequantize_rows(const int8_t* codes, const float* scales, size_t rows, size_t row_len,
                               uint32_t block, void* out, qar_dtype out_dtype, void* stream) {
    RowShape sh;
    qar_status st = row_shape(rows, row_len, block, sh);
    if (st != QAR_OK || sh.n == 0) return st;
    if (!codes || !scales || !out) return QAR_ERR_INVALID_ARG;
    if (!dtype_ok(out_dtype)) return QAR_ERR_UNSUPPORTED;
    if (flat_ok(sh, block) && aligned(codes, 16) && aligned(out, 16))
        return qar_dequantize(codes, scales, sh.n, block, out, out_dtype, stream);
    if (!aligned(out, dtype_bytes(out_dtype)) || !aligned(scales, 4)) return QAR_ERR_MISALIGNED;
    const Range ci = range(codes, sh.n), si = range(scales, sh.nblocks * 4),
                oo = range(out, sh.n * dtype_bytes(out_dtype));
    if (overlap(oo, ci) || overlap(oo, si)) return QAR_ERR_INVALID_ARG;
    qar::RowsCall c = rows_call(qar::kRowsDequantize, sh, block);
    c.vector = sh.row_len % 16 == 0 && aligned(codes, 16) && aligned(out, 16);
    c.kind = out_dtype == QAR_BF16 ? qar::kInBF16 : qar::kInF32;
    c.codes_in = codes;
    c.scales_in = scales;
    c.out = out;
    const hipError_t e = qar::launch_rows(c, (hipStream_t)stream);
    return e == hipSuccess ? QAR_OK : hip_fail(e, "qar_dequantize_rows");
}

qar_status qar_reduce_quantized_rows(const int8_t* const* codes, const float* const* scales, uint32_t nranks,
                                     size_t rows, size_t row_len, uint32_t block, int8_t* codes_out,
                                     float* scales_out, void* out, qar_dtype out_dtype, void* stream) {
    RowShape sh;
    qar_status st = row_shape(rows, row_len, block, sh);
    if (st != QAR_OK || sh.n == 0) return st;
    if (!codes || !scales || !codes_out || !scales_out) return QAR_ERR_INVALID_ARG;
    if (nranks == 0 || nranks > QAR_MAX_RANKS) return QAR_ERR_INVALID_ARG;
    if (out && !dtype_ok(out_dtype)) return QAR_ERR_UNSUPPORTED;
    if (flat_ok(sh, block)) {
        bool al = aligned(codes_out, 16) && (!out || aligned(out, 16));
        for (uint32_t r = 0; al && r < nranks; ++r) al = codes[r] && aligned(codes[r], 16);
        if (al)
            return qar_reduce_quantized(codes, scales, nranks, sh.n, block, codes_out, scales_out, out, out_dtype,
                                        stream);
    }
    if (!aligned(scales_out, 4) || (out && !aligned(out, dtype_bytes(out_dtype)))) return QAR_ERR_MISALIGNED;
    const Range co = range(codes_out, sh.n), so = range(scales_out, sh.nblocks * 4);
    if (overlap(co, so)) return QAR_ERR_INVALID_ARG;
    Range oo{0, 0};
    if (out) {
        oo = range(out, sh.n * dtype_bytes(out_dtype));
        if (overlap(oo, co) || overlap(oo, so)) return QAR_ERR_INVALID_ARG;
    }
    qar::RowsCall c = rows_call(qar::kRowsReduce, sh, block);
    int same_codes = -1, same_scales = -1;
    for (uint32_t r = 0; r < nranks; ++r) {
        if (!codes[r] || !scales[r]) return QAR_ERR_INVALID_ARG;
        if (!aligned(scales[r], 4)) return QAR_ERR_MISALIGNED;
        const Range ci = range(codes[r], sh.n), si = range(scales[r], sh.nblocks * 4);
        if (bad_overlap(co, ci, true) || bad_overlap(so, si, true) || overlap(co, si) || overlap(so, ci))
            return QAR_ERR_INVALID_ARG;
        if (out && (overlap(oo, ci) || overlap(oo, si))) return QAR_ERR_INVALID_ARG;
        if (co.lo == ci.lo) same_codes = (int)r;
        if (so.lo == si.lo) same_scales = (int)r;
        c.rp.codes[r] = codes[r];
        c.rp.scales[r] = scales[r];
    }
    if (same_codes != same_scales) return QAR_ERR_INVALID_ARG;
    c.vector = sh.row_len % 16 == 0 && aligned(codes_out, 16) && (!out || aligned(out, 16));
    for (uint32_t r = 0; c.vector && r < nranks; ++r) c.vector = aligned(codes[r], 16);
    c.kind = (out && out_dtype == QAR_F32) ? qar::kInF32 : qar::kInBF16;
    c.nranks = (int)nranks;
    c.codes_out = codes_out;
    c.scales_out = scales_out;
    c.out = out;
    const hipError_t e = qar::launch_rows(c, (hipStream_t)stream);
    return e == hipSuccess ? QAR_OK : hip_fail(e, "qar_reduce_quantized_rows");
}

qar_status qar_ring_step_rows(const int8_t* codes_in, const float* scales_in, const void* local, qar_dtype dtype,
                              size_t rows, size_t row_len, uint32_t block, int8_t* codes_out, float* scales_out,
                              void* stream) {
    RowShape sh;
    qar_status st = row_shape(rows, row_len, block, sh);
    if (st != QAR_OK || sh.n == 0) return st;
    if (!codes_in || !scales_in || !local || !codes_out || !scales_out) return QAR_ERR_INVALID_ARG;
    if (!dtype_ok(dtype)) return QAR_ERR_UNSUPPORTED;
    if (flat_ok(sh, block) && aligned(codes_in, 16) && aligned(codes_out, 16) && aligned(local, 16))
        return qar_ring_step(codes_in, scales_in, local, dtype, sh.n, block, codes_out, scales_out, stream);
    if (!aligned(local, dtype_bytes(dtype)) || !aligned(scales_in, 4) || !aligned(scales_out, 4))
        return QAR_ERR_MISALIGNED;
    const Range ci = range(codes_in, sh.n), si = range(scales_in, sh.nblocks * 4),
                li = range(local, sh.n * dtype_bytes(dtype)), co = range(codes_out, sh.n),
                so = range(scales_out, sh.nblocks * 4);
    if (bad_overlap(co, ci, true) || bad_overlap(so, si, true) || overlap(co, si) || overlap(so, ci) ||
        overlap(co, li) || overlap(so, li) || overlap(co, so))
        return QAR_ERR_INVALID_ARG;
    if ((co.lo == ci.lo) != (so.lo == si.lo)) return QAR_ERR_INVALID_ARG;
    qar::RowsCall c = rows_call(qar::kRowsRingStep, sh, block);
    c.vector = sh.row_len % 16 == 0 && aligned(codes_in, 16) && aligned(codes_out, 16) && aligned(local, 16);
    c.kind = dtype == QAR_BF16 ? qar::kInBF16 : qar::kInF32;
    c.x = local;
    c.codes_in = codes_in;
    c.scales_in = scales_in;
    c.codes_out = codes_out;
    c.scales_out = scales_out;
    const hipError_t e = qar::launch_rows(c, (hipStream_t)stream);
    return e == hipSuccess ? QAR_OK : hip_fail(e, "qar_ring_step_rows");
}

} // extern "C"
