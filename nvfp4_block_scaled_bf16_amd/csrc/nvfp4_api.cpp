// nvfp4_api.cpp -- the C ABI of libnvfp4 (declared in include/nvfp4.h):
// host-side validation, then stream-ordered launches.  Nothing is enqueued
// unless every check passes; the library allocates no memory.
#include "nvfp4.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <atomic>
#include <mutex>
#include <string>
#include <vector>

#include "nvfp4_device.hpp"
#include "nvfp4_internal.h"

using namespace nvfp4;

namespace {

thread_local std::string g_last_error;

nvfp4_status fail(nvfp4_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

nvfp4_status ok() {
    g_last_error.clear();
    return NVFP4_OK;
}

nvfp4_status check_hip(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(NVFP4_EDEVICE, "%s: %s", what, hipGetErrorString(e));
    return NVFP4_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct Dir {
    bool want;
    nvfp4_status st;
};

// a direction is requested when any of its pointers is given; then all of
// them must be given
Dir direction(const char* name, const void* q, const void* sf, const void* amax) {
    int given = (q != nullptr) + (sf != nullptr) + (amax != nullptr);
    if (given == 0) return {false, NVFP4_OK};
    if (given != 3) return {true, fail(NVFP4_EINVAL, "%s output: q, sf and amax must all be given (or all NULL)", name)};
    if (!aligned(q, 16)) return {true, fail(NVFP4_EALIGN, "%s_q must be 16-byte aligned", name)};
    if (!aligned(amax, 4)) return {true, fail(NVFP4_EALIGN, "%s_amax must be 4-byte aligned", name)};
    return {true, NVFP4_OK};
}

nvfp4_status check_shape(int64_t M, int64_t K, bool row, bool col, int mode) {
    if (M < 0 || K < 0) return fail(NVFP4_EINVAL, "negative size M=%lld K=%lld", (long long)M, (long long)K);
    if (row && K % 16 != 0) return fail(NVFP4_ESHAPE, "rowwise output needs K %% 16 == 0 (K=%lld)", (long long)K);
    if (col && M % 16 != 0) return fail(NVFP4_ESHAPE, "columnwise output needs M %% 16 == 0 (M=%lld)", (long long)M);
    if (col && K % 8 != 0) return fail(NVFP4_ESHAPE, "columnwise output needs K %% 8 == 0 (K=%lld)", (long long)K);
    if (mode == NVFP4_TILE_16x16 && (M % 16 != 0 || K % 16 != 0))
        return fail(NVFP4_ESHAPE, "16x16 tiles need M and K multiples of 16 (M=%lld K=%lld)", (long long)M, (long long)K);
    if (M > (int64_t(1) << 40)) return fail(NVFP4_ESHAPE, "M too large (M=%lld)", (long long)M);
    // the encoding kernel addresses 32 rows of x with 32-bit offsets
    if (K >= kMaxEncodeK) return fail(NVFP4_ESHAPE, "K must be below %lld (K=%lld)", (long long)kMaxEncodeK, (long long)K);
    return NVFP4_OK;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

GroupTable empty_table() {
    GroupTable gt;
    gt.n = 0;
    gt.first = 0;
    return gt;
}

// one-shot timing events set by nvfp4_trace_encode (hipEvent_t, caller-owned)
thread_local hipEvent_t g_trace_before = nullptr;
thread_local hipEvent_t g_trace_after = nullptr;

// launch an encoding kernel with the pending trace events if any: the
// kernel's dispatch records them at its start and end
template <class Launch>
nvfp4_status encode_launch(Launch&& launch) {
    hipEvent_t before = g_trace_before, after = g_trace_after;
    g_trace_before = g_trace_after = nullptr;
    return check_hip(launch(before, after), "encode");
}

// ------------------------------------------------------ per-device state
//
// Per device, set up on first use: the compute-unit count (grids of the
// persistent kernels), the counts of the cross-workgroup wait slots (see
// SyncArg: slots are handed out in turn, each advanced by its launch's
// arrivals), and a word of pinned host memory, visible to the device, where
// a wait that gave up records the failure; every call that takes a slot
// checks it first and reports NVFP4_EDEVICE once for such a failure.
struct DeviceState {
    bool init = false;
    int cus = 0;
    uint64_t next_slot = 0;
    uint64_t slot_count[kSyncSlots] = {};
    unsigned int* err_host = nullptr;
    unsigned int* err_dev = nullptr;
};
std::mutex g_dev_mu;
std::vector<DeviceState> g_dev;
// nvfp4_test_fail_next_wait: the next slot handed out gets a base no launch
// reaches (its waits give up at their bound)
std::atomic<bool> g_fail_next_wait{false};

nvfp4_status stream_device(hipStream_t st, int* dev) {
    hipError_t e = st ? hipStreamGetDevice(st, dev) : hipGetDevice(dev);
    return e == hipSuccess ? NVFP4_OK : fail(NVFP4_EDEVICE, "stream device: %s", hipGetErrorString(e));
}

// call with g_dev_mu held; with_err: also the pinned error word (only the
// launches with waits need it, and those are never made under capture)
nvfp4_status device_init(int dev, DeviceState** out, bool with_err = false) {
    if ((int)g_dev.size() <= dev) g_dev.resize(dev + 1);
    DeviceState& d = g_dev[dev];
    hipError_t e;
    if (!d.init) {
        int n = 0;
        if ((e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess || n <= 0)
            return fail(NVFP4_EDEVICE, "device attribute: %s", hipGetErrorString(e));
        d.cus = n;
        d.init = true;
    }
    if (with_err && d.err_host == nullptr) {
        void* h = nullptr;
        if ((e = hipHostMalloc(&h, sizeof(unsigned int), hipHostMallocMapped)) != hipSuccess)
            return fail(NVFP4_EDEVICE, "pinned error word: %s", hipGetErrorString(e));
        void* dp = nullptr;
        if ((e = hipHostGetDevicePointer(&dp, h, 0)) != hipSuccess) {
            (void)hipHostFree(h);
            return fail(NVFP4_EDEVICE, "pinned error word: %s", hipGetErrorString(e));
        }
        *static_cast<unsigned int*>(h) = 0u;
        d.err_dev = static_cast<unsigned int*>(dp);
        d.err_host = static_cast<unsigned int*>(h);
    }
    *out = &d;
    return NVFP4_OK;
}

nvfp4_status device_cus(hipStream_t st, int* cus) {
    int dev = 0;
    nvfp4_status s = stream_device(st, &dev);
    if (s != NVFP4_OK) return s;
    std::lock_guard<std::mutex> lock(g_dev_mu);
    DeviceState* d = nullptr;
    if ((s = device_init(dev, &d)) != NVFP4_OK) return s;
    *cus = d->cus;
    return NVFP4_OK;
}

// Launches with cross-workgroup waits take their slot's base count from the
// host at the call, so they must not be recorded into a graph (a replay would
// reuse the recorded base).  On a capturing stream the library takes the
// paths without waits instead (a fill launch before the amax pass, the
// two-launch schedule).
bool capturing(hipStream_t st) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    return hipStreamIsCapturing(st, &cs) == hipSuccess && cs != hipStreamCaptureStatusNone;
}

// A slot for a launch of `arrivals` arrivals on stream st.
struct SyncTicket {
    SyncArg arg;
    int dev;
    uint64_t arrivals;
};

nvfp4_status sync_take(hipStream_t st, uint64_t arrivals, SyncTicket* t) {
    int dev = 0;
    nvfp4_status s = stream_device(st, &dev);
    if (s != NVFP4_OK) return s;
    std::lock_guard<std::mutex> lock(g_dev_mu);
    DeviceState* d = nullptr;
    if ((s = device_init(dev, &d, true)) != NVFP4_OK) return s;
    if (__atomic_load_n(d->err_host, __ATOMIC_ACQUIRE) != 0u) {
        __atomic_store_n(d->err_host, 0u, __ATOMIC_RELEASE);
        return fail(NVFP4_EDEVICE, "an earlier call's cross-workgroup wait gave up (its outputs are invalid)");
    }
    const int slot = (int)(d->next_slot++ % kSyncSlots);
    t->arg.slot = slot;
    t->arg.base = d->slot_count[slot];
    if (g_fail_next_wait.exchange(false)) t->arg.base += (uint64_t)1 << 40;
    t->arg.err = d->err_dev;
    t->dev = dev;
    t->arrivals = arrivals;
    d->slot_count[slot] += arrivals;
    return NVFP4_OK;
}

// the launch holding ticket t did not start: its arrivals never come
void sync_return(const SyncTicket& t) {
    std::lock_guard<std::mutex> lock(g_dev_mu);
    g_dev[t.dev].slot_count[t.arg.slot] -= t.arrivals;
}

// Amax launch whose first workgroups zero its outputs (a[0..na), b[0..nb))
// before the others combine into them, in place of a separate fill launch.
// The zeroing workgroups must exist: the grid has at least that many.
nvfp4_status amax_zero_first(int kind, const uint16_t* x, int64_t K, int64_t row_begin, int64_t row_end,
                             float* row_amax, float* col_amax, float* t0, float* t1, const GroupTable& gt,
                             float* a, int64_t na, float* b, int64_t nb, hipStream_t st) {
    if (a == nullptr) na = 0;
    if (b == nullptr) nb = 0;
    ZeroFirst z{a, na, b, nb, (int)((na + nb + kZeroPerWg - 1) / kZeroPerWg)};
    if (z.wgs == 0 || z.wgs > amax_grid_size(kind, K, row_begin, row_end) || capturing(st)) {
        // nothing to zero, more than the grid has workgroups, or a capture: a fill launch
        nvfp4_status s = check_hip(launch_fill2(a, na, b, nb, 0.0f, st), "fill");
        if (s != NVFP4_OK) return s;
        return check_hip(launch_amax(kind, x, K, row_begin, row_end, row_amax, col_amax, t0, t1, gt, st), "amax");
    }
    SyncTicket tk;
    nvfp4_status s = sync_take(st, (uint64_t)z.wgs, &tk);
    if (s != NVFP4_OK) return s;
    s = check_hip(launch_amax(kind, x, K, row_begin, row_end, row_amax, col_amax, t0, t1, gt, st, z, tk.arg), "amax");
    if (s != NVFP4_OK) sync_return(tk);
    return s;
}

// Rowwise-only per-token casts are served by the single-pass row kernel
// when K is within its rounds (K <= 65536).  Grid: one workgroup per batch
// (up to 2^20 of them, then persistent over the rest): at 16384 x 8192 the
// dispatcher's balancing of 4096 one-batch workgroups beat two persistent
// workgroups per compute unit (8 batches each), 55.8-56.2 us against
// 58.4-59.6 us; 1024 to 3072 workgroups measured in between.
bool rows_path(int64_t K) { return rows_rounds(K) != 0; }

unsigned rows_grid(int cus, int64_t M, int64_t K) {
    (void)cus;
    const int64_t nb = rows_batches(M, K);
    const int64_t cap = (int64_t)1 << 20;
    return (unsigned)(nb < cap ? nb : cap);
}

// zero-fill up to two fp32 arrays (one launch) before an atomic-max pass
nvfp4_status zero(float* a, int64_t na, float* b, int64_t nb, hipStream_t st) {
    return check_hip(launch_fill2(a, na, b, nb, 0.0f, st), "fill");
}

// ------------------------------------------------------- cast schedules

std::atomic<int> g_schedule{NVFP4_SCHEDULE_AUTO};

// Resident schedule of an M x K cast: a grid of ceil(K / 256) strips x nband
// bands, every workgroup resident at once (cap of them fit), each owning a
// run of up to `run` 256-row tiles; runs over 32 tiles are not offered.
struct ResPlan {
    int run = 0, nband = 0;
    unsigned grid = 0;   // 0: the schedule does not apply
};

ResPlan resident_plan(int cap, int64_t M, int64_t K) {
    ResPlan p;
    const int64_t tx = (K + 255) / 256, ty = (M + 255) / 256;
    // (the columnwise output is addressed with 32-bit offsets)
    if (cap <= 0 || M <= 0 || K <= 0 || tx > cap || M / 2 * K >= ((int64_t)1 << 31)) return p;
    const int64_t per = cap / tx;
    const int64_t run = (ty + per - 1) / per;
    if (run > 32) return p;
    p.run = (int)run;
    p.nband = (int)((ty + run - 1) / run);
    p.grid = (unsigned)(tx * p.nband);
    return p;
}

// the plan for this call under the current schedule (grid 0: two passes)
nvfp4_status resident_choice(int emode, bool row, bool col, int64_t M, int64_t K, hipStream_t st, ResPlan* out) {
    *out = ResPlan{};
    if (g_schedule.load(std::memory_order_relaxed) == NVFP4_SCHEDULE_TWO_PASS || capturing(st)) return NVFP4_OK;
    int cus = 0;
    nvfp4_status s = device_cus(st, &cus);
    if (s != NVFP4_OK) return s;
    const ResPlan p = resident_plan(resident_blocks_per_cu(emode, row, col) * cus, M, K);
    // Automatic: resident when every workgroup keeps its whole run (at most
    // two tiles) in registers, so that x is read once.  Longer runs re-read
    // all but two tiles per workgroup, and the encoding phase, with two
    // waves per SIMD and all the vector work of the cast, then takes longer
    // than the separate encoding pass.
    if (g_schedule.load(std::memory_order_relaxed) == NVFP4_SCHEDULE_RESIDENT || p.run <= 2) *out = p;
    return NVFP4_OK;
}

// One launch: zero-first of the amax outputs, amax phase, grid-wide wait,
// encoding phase (with the calibration update when cal.buf is set).
nvfp4_status resident_cast(int emode, const uint16_t* x, int64_t M, int64_t K, uint8_t* rq, uint8_t* rsf, float* ra,
                           uint8_t* cq, uint8_t* csf, float* ca, const Calib& cal, const ResPlan& p, hipStream_t st) {
    const bool tok = emode == ENC_TOKEN;
    const int64_t na = ra ? (tok ? M : 1) : 0, nb = ca ? (tok ? K : 1) : 0;
    ZeroFirst z{ra, na, ca, nb, (int)((na + nb + kZeroPerWg - 1) / kZeroPerWg)};
    nvfp4_status s;
    if ((unsigned)z.wgs > p.grid) {
        // more zeroing than workgroups: a fill launch first
        if ((s = zero(ra, na, ca, nb, st)) != NVFP4_OK) return s;
        z.wgs = 0;
    }
    ResArgs a{x, M, K, ra, ca, rq, rsf, cq, csf, p.run, p.nband, z, SyncArg{0ull, nullptr, -1},
              SyncArg{0ull, nullptr, -1}, cal};
    SyncTicket zt{}, bt{};
    if (z.wgs > 0) {
        if ((s = sync_take(st, (uint64_t)z.wgs, &zt)) != NVFP4_OK) return s;
        a.zsync = zt.arg;
    }
    if ((s = sync_take(st, p.grid, &bt)) != NVFP4_OK) {
        if (z.wgs > 0) sync_return(zt);
        return s;
    }
    a.bar = bt.arg;
    s = encode_launch([&](hipEvent_t b, hipEvent_t e) {
        return launch_resident(emode, ra != nullptr, ca != nullptr, a, p.grid, st, b, e);
    });
    if (s != NVFP4_OK) {
        sync_return(bt);
        if (z.wgs > 0) sync_return(zt);
    }
    return s;
}

// cal_buf (may be null): buf[0] = max(buf[0] * decay, tensor amax), done by
// the encoding kernel from the amax it has just read
// stochastic rounding of the element codes (nvfp4_quantize_sr)
struct Rounding {
    bool stochastic;
    uint64_t seed;
    uint32_t offset;
};

nvfp4_status quantize_impl(const void* xv, int64_t M, int64_t K, nvfp4_scaling mode,
                           uint8_t* row_q, uint8_t* row_sf, float* row_amax,
                           uint8_t* col_q, uint8_t* col_sf, float* col_amax, void* stream,
                           float* cal_buf = nullptr, float decay = 0.0f,
                           Rounding rounding = Rounding{false, 0, 0}, bool swizzled = false) {
    if (mode != NVFP4_PER_TENSOR && mode != NVFP4_PER_TOKEN && mode != NVFP4_TILE_16x16)
        return fail(NVFP4_EINVAL, "unknown scaling mode %d", (int)mode);
    if (rounding.stochastic && mode == NVFP4_TILE_16x16)
        return fail(NVFP4_EINVAL, "stochastic rounding is offered for per-tensor and per-token scaling only");
    Dir r = direction("row", row_q, row_sf, row_amax);
    if (r.st != NVFP4_OK) return r.st;
    Dir c = direction("col", col_q, col_sf, col_amax);
    if (c.st != NVFP4_OK) return c.st;
    if (!r.want && !c.want) return fail(NVFP4_EINVAL, "no output direction requested");
    nvfp4_status s = check_shape(M, K, r.want, c.want, mode);
    if (s != NVFP4_OK) return s;
    if (rounding.stochastic && M >= ((int64_t)1 << 32))
        return fail(NVFP4_ESHAPE, "stochastic rounding needs M < 2^32 (M = %lld)", (long long)M);
    if (swizzled) {
        if (mode == NVFP4_TILE_16x16) return fail(NVFP4_EINVAL, "swizzled scales are offered for per-tensor and per-token scaling only");
        if (M % 128 != 0 || K % 128 != 0)
            return fail(NVFP4_ESHAPE, "swizzled scales need M %% 128 == 0 and K %% 128 == 0 (M=%lld K=%lld)", (long long)M, (long long)K);
        if (M * (K / 16) >= ((int64_t)1 << 31)) return fail(NVFP4_ESHAPE, "swizzled scales need M * K / 16 < 2^31");
        if ((r.want && !aligned(row_sf, 4)) || (c.want && !aligned(col_sf, 4)))
            return fail(NVFP4_EALIGN, "swizzled scales must be 4-byte aligned");
    }
    if (xv == nullptr && M > 0 && K > 0) return fail(NVFP4_EINVAL, "x is NULL");
    if (!aligned(xv, 16)) return fail(NVFP4_EALIGN, "x must be 16-byte aligned");
    const uint16_t* x = static_cast<const uint16_t*>(xv);
    hipStream_t st = as_stream(stream);
    float* ra = r.want ? row_amax : nullptr;
    float* ca = c.want ? col_amax : nullptr;
    const GroupTable gt = empty_table();

    if (cal_buf && (M == 0 || K == 0)) {
        // nothing observed: buf = max(buf * decay, 0)
        if ((s = check_hip(launch_accumulate_reduce(cal_buf, nullptr, 0, decay, st), "calibration")) != NVFP4_OK) return s;
    }
    // what the calibration observes: the tensor amax, as the max of the
    // per-column (else per-row) vector, or the per-tensor value
    Calib cal{cal_buf, nullptr, 0, decay};
    if (cal_buf) {
        if (mode == NVFP4_PER_TOKEN) { cal.obs = ca ? ca : ra; cal.n = ca ? K : M; }
        else { cal.obs = ra ? ra : ca; cal.n = 1; }
    }
    if (mode == NVFP4_PER_TOKEN && r.want && !c.want && M > 0 && K > 0 && !rounding.stochastic && !swizzled &&
        rows_path(K) && g_schedule.load(std::memory_order_relaxed) != NVFP4_SCHEDULE_RESIDENT) {
        // rowwise only: each row's amax is found and used on chip, x is read
        // once
        int cus = 0;
        if ((s = device_cus(st, &cus)) != NVFP4_OK) return s;
        const unsigned grid = rows_grid(cus, M, K);
        if ((s = encode_launch([&](hipEvent_t b, hipEvent_t a) {
                 return launch_rows(x, M, K, row_q, row_sf, ra, grid, st, b, a);
             })) != NVFP4_OK)
            return s;
        if (cal_buf && (s = check_hip(launch_accumulate_reduce(cal_buf, ra, M, decay, st), "calibration")) != NVFP4_OK)
            return s;
        return ok();
    }
    if ((mode == NVFP4_PER_TOKEN || mode == NVFP4_PER_TENSOR) && M > 0 && K > 0 && !rounding.stochastic && !swizzled) {
        // amax and encoding in one resident launch, where it applies
        const int emode = mode == NVFP4_PER_TOKEN ? ENC_TOKEN : ENC_TENSOR;
        ResPlan p;
        if ((s = resident_choice(emode, r.want, c.want, M, K, st, &p)) != NVFP4_OK) return s;
        if (p.grid != 0) {
            s = resident_cast(emode, x, M, K, r.want ? row_q : nullptr, r.want ? row_sf : nullptr, ra,
                              c.want ? col_q : nullptr, c.want ? col_sf : nullptr, ca, cal, p, st);
            return s != NVFP4_OK ? s : ok();
        }
    }
    if (mode == NVFP4_PER_TOKEN) {
        if (M == 0 || K == 0) return zero(ra, M, ca, K, st) != NVFP4_OK ? NVFP4_EDEVICE : ok();
        if ((s = amax_zero_first(AMAX_TOKEN, x, K, 0, M, ra, ca, nullptr, nullptr, gt, ra, M, ca, K, st)) != NVFP4_OK)
            return s;
        if (rounding.stochastic)
            s = encode_launch([&](hipEvent_t b, hipEvent_t a) { return launch_encode_sr(ENC_TOKEN, r.want, c.want, x, M, K, ra, ca, row_q, row_sf,
                                  col_q, col_sf, rounding.seed, rounding.offset, st, b, a); });
        else
            s = encode_launch([&](hipEvent_t b, hipEvent_t a) { return launch_encode(ENC_TOKEN, r.want, c.want, false, x, M, K, 0, M, ra, ca, row_q, row_sf, col_q, col_sf,
                                  nullptr, nullptr, gt, st, b, a, cal, swizzled); });
        return s != NVFP4_OK ? s : ok();
    }
    // per-tensor and 16x16 tiles: one tensor amax
    if (M == 0 || K == 0)
        return zero(ra, ra ? (mode == NVFP4_TILE_16x16 ? M : 1) : 0, ca, ca ? (mode == NVFP4_TILE_16x16 ? K : 1) : 0, st) != NVFP4_OK
                   ? NVFP4_EDEVICE : ok();
    // the tensor amax is combined into entry 0 of each vector (16x16 tiles
    // fill the rest of theirs from it in the encoding kernel)
    if ((s = amax_zero_first(AMAX_TENSOR, x, K, 0, M, nullptr, nullptr, ra, ca, gt, ra, ra ? 1 : 0, ca, ca ? 1 : 0, st)) !=
        NVFP4_OK)
        return s;
    const int emode = mode == NVFP4_TILE_16x16 ? ENC_TILE : ENC_TENSOR;
    if (rounding.stochastic) {
        s = encode_launch([&](hipEvent_t b, hipEvent_t a) { return launch_encode_sr(ENC_TENSOR, r.want, c.want, x, M, K, ra, ca, row_q, row_sf,
                              col_q, col_sf, rounding.seed, rounding.offset, st, b, a); });
        return s != NVFP4_OK ? s : ok();
    }
    if ((s = encode_launch([&](hipEvent_t b, hipEvent_t a) { return launch_encode(emode, r.want, c.want, false, x, M, K, 0, M, ra, ca, row_q, row_sf, col_q, col_sf,
                                     emode == ENC_TILE ? ra : nullptr, emode == ENC_TILE ? ca : nullptr, gt, st, b, a, cal,
                                     swizzled); })) != NVFP4_OK)
        return s;
    return ok();
}

}  // namespace

extern "C" {

int nvfp4_abi_version(void) { return NVFP4_ABI_VERSION; }

const char* nvfp4_last_error(void) { return g_last_error.c_str(); }

nvfp4_status nvfp4_trace_encode(void* before, void* after) {
    if ((before == nullptr) != (after == nullptr)) return fail(NVFP4_EINVAL, "give both trace events or neither");
    g_trace_before = static_cast<hipEvent_t>(before);
    g_trace_after = static_cast<hipEvent_t>(after);
    return ok();
}

nvfp4_status nvfp4_test_fail_next_wait(void) {
    g_fail_next_wait.store(true);
    return ok();
}

nvfp4_status nvfp4_set_schedule(nvfp4_schedule schedule) {
    const int v = (int)schedule;
    if (v != NVFP4_SCHEDULE_AUTO && v != NVFP4_SCHEDULE_TWO_PASS && v != NVFP4_SCHEDULE_RESIDENT)
        return fail(NVFP4_EINVAL, "unknown schedule %d", v);
    g_schedule.store(v, std::memory_order_relaxed);
    return ok();
}

nvfp4_status nvfp4_quantize(const void* x, int64_t M, int64_t K, nvfp4_scaling mode,
                            uint8_t* row_q, uint8_t* row_sf, float* row_amax,
                            uint8_t* col_q, uint8_t* col_sf, float* col_amax, void* stream) {
    return quantize_impl(x, M, K, mode, row_q, row_sf, row_amax, col_q, col_sf, col_amax, stream);
}

nvfp4_status nvfp4_quantize_swizzled(const void* x, int64_t M, int64_t K, nvfp4_scaling mode,
                                     uint8_t* row_q, uint8_t* row_sf, float* row_amax,
                                     uint8_t* col_q, uint8_t* col_sf, float* col_amax, void* stream) {
    return quantize_impl(x, M, K, mode, row_q, row_sf, row_amax, col_q, col_sf, col_amax, stream, nullptr, 0.0f,
                         Rounding{false, 0, 0}, true);
}

nvfp4_status nvfp4_quantize_calibrate(const void* x, int64_t M, int64_t K, nvfp4_scaling mode,
                                      uint8_t* row_q, uint8_t* row_sf, float* row_amax,
                                      uint8_t* col_q, uint8_t* col_sf, float* col_amax,
                                      float* buf, float decay, void* stream) {
    if (!buf) return fail(NVFP4_EINVAL, "buf is NULL");
    if (!aligned(buf, 4)) return fail(NVFP4_EALIGN, "buf must be 4-byte aligned");
    if (!(decay >= 0.0f && decay <= 1.0f)) return fail(NVFP4_EINVAL, "decay must lie in [0, 1]");
    return quantize_impl(x, M, K, mode, row_q, row_sf, row_amax, col_q, col_sf, col_amax, stream, buf, decay);
}

nvfp4_status nvfp4_quantize_sr(const void* x, int64_t M, int64_t K, nvfp4_scaling mode,
                               uint8_t* row_q, uint8_t* row_sf, float* row_amax,
                               uint8_t* col_q, uint8_t* col_sf, float* col_amax,
                               uint64_t seed, uint32_t offset, void* stream) {
    return quantize_impl(x, M, K, mode, row_q, row_sf, row_amax, col_q, col_sf, col_amax, stream, nullptr, 0.0f,
                         Rounding{true, seed, offset});
}

nvfp4_status nvfp4_quantize_rht(const void* xv, int64_t M, int64_t K, nvfp4_scaling mode, uint32_t sign_mask,
                                uint8_t* row_q, uint8_t* row_sf, float* row_amax,
                                uint8_t* col_q, uint8_t* col_sf, float* col_amax, void* stream) {
    if (mode != NVFP4_PER_TENSOR && mode != NVFP4_PER_TOKEN)
        return fail(NVFP4_EINVAL, "the Hadamard transform is offered for per-tensor and per-token scaling only");
    if (sign_mask > 0xFFFFu) return fail(NVFP4_EINVAL, "sign_mask has 16 bits (got %#x)", sign_mask);
    Dir c = direction("col", col_q, col_sf, col_amax);
    if (c.st != NVFP4_OK) return c.st;
    if (!c.want) return fail(NVFP4_EINVAL, "the Hadamard transform applies to the columnwise output, which must be given");
    Dir r = direction("row", row_q, row_sf, row_amax);
    if (r.st != NVFP4_OK) return r.st;
    nvfp4_status s = check_shape(M, K, r.want, true, mode);
    if (s != NVFP4_OK) return s;
    if (M > (int64_t)65535 * 128) return fail(NVFP4_ESHAPE, "the Hadamard transform needs M <= 65535 * 128 (M=%lld)", (long long)M);
    if (xv == nullptr && M > 0 && K > 0) return fail(NVFP4_EINVAL, "x is NULL");
    if (!aligned(xv, 16)) return fail(NVFP4_EALIGN, "x must be 16-byte aligned");
    hipStream_t st = as_stream(stream);
    const bool tok = mode == NVFP4_PER_TOKEN;
    float* ra = r.want ? row_amax : nullptr;
    const int64_t na = tok ? K : 1, nb = ra ? (tok ? M : 1) : 0;
    if (M == 0 || K == 0) return (s = zero(col_amax, na, ra, nb, st)) != NVFP4_OK ? s : ok();
    // the amax launch's first workgroups zero its outputs (a fill launch
    // instead under stream capture, or when the grid is too small for them)
    ZeroFirst z{col_amax, na, ra, nb, (int)((na + nb + kZeroPerWg - 1) / kZeroPerWg)};
    SyncTicket tk;
    const bool zero_first = z.wgs <= rht_amax_grid_size(M, K) && !capturing(st);
    if (zero_first) {
        if ((s = sync_take(st, (uint64_t)z.wgs, &tk)) != NVFP4_OK) return s;
    } else if ((s = zero(col_amax, na, ra, nb, st)) != NVFP4_OK) {
        return s;
    }
    const uint16_t* x = static_cast<const uint16_t*>(xv);
    bool amax_launched = false;
    s = encode_launch([&](hipEvent_t b, hipEvent_t a) {
        return launch_rht(tok ? ENC_TOKEN : ENC_TENSOR, x, M, K, sign_mask, ra, col_amax, r.want ? row_q : nullptr,
                          r.want ? row_sf : nullptr, col_q, col_sf, st, b, a,
                          zero_first ? z : ZeroFirst{nullptr, 0, nullptr, 0, 0},
                          zero_first ? tk.arg : SyncArg{0ull, nullptr, -1}, &amax_launched);
    });
    if (zero_first && !amax_launched) sync_return(tk);
    return s != NVFP4_OK ? s : ok();
}

nvfp4_status nvfp4_quantize_rowwise(const void* x, int64_t M, int64_t K, nvfp4_scaling mode,
                                    uint8_t* row_q, uint8_t* row_sf, float* row_amax, void* stream) {
    if (!row_q || !row_sf || !row_amax) return fail(NVFP4_EINVAL, "rowwise outputs must not be NULL");
    return quantize_impl(x, M, K, mode, row_q, row_sf, row_amax, nullptr, nullptr, nullptr, stream);
}

nvfp4_status nvfp4_quantize_columnwise(const void* x, int64_t M, int64_t K, nvfp4_scaling mode,
                                       uint8_t* col_q, uint8_t* col_sf, float* col_amax, void* stream) {
    if (!col_q || !col_sf || !col_amax) return fail(NVFP4_EINVAL, "columnwise outputs must not be NULL");
    return quantize_impl(x, M, K, mode, nullptr, nullptr, nullptr, col_q, col_sf, col_amax, stream);
}

nvfp4_status nvfp4_amax(const void* xv, int64_t M, int64_t K, nvfp4_scaling mode,
                        float* row_amax, float* col_amax, void* stream) {
    if (mode != NVFP4_PER_TENSOR && mode != NVFP4_PER_TOKEN)
        return fail(NVFP4_EINVAL, "nvfp4_amax takes PER_TENSOR or PER_TOKEN (mode %d)", (int)mode);
    if (!row_amax && !col_amax) return fail(NVFP4_EINVAL, "no amax output given");
    if ((row_amax && !aligned(row_amax, 4)) || (col_amax && !aligned(col_amax, 4)))
        return fail(NVFP4_EALIGN, "amax outputs must be 4-byte aligned");
    if (M < 0 || K < 0) return fail(NVFP4_EINVAL, "negative size");
    if (K % 8 != 0) return fail(NVFP4_ESHAPE, "nvfp4_amax needs K %% 8 == 0 (K=%lld)", (long long)K);
    if (K >= kMaxEncodeK) return fail(NVFP4_ESHAPE, "K must be below %lld (K=%lld)", (long long)kMaxEncodeK, (long long)K);
    if (!xv) return fail(NVFP4_EINVAL, "x is NULL");
    if (!aligned(xv, 16)) return fail(NVFP4_EALIGN, "x must be 16-byte aligned");
    const uint16_t* x = static_cast<const uint16_t*>(xv);
    hipStream_t st = as_stream(stream);
    const GroupTable gt = empty_table();
    nvfp4_status s;
    if (mode == NVFP4_PER_TOKEN) {
        if (M == 0 || K == 0) return zero(row_amax, M, col_amax, K, st) != NVFP4_OK ? NVFP4_EDEVICE : ok();
        if ((s = amax_zero_first(AMAX_TOKEN, x, K, 0, M, row_amax, col_amax, nullptr, nullptr, gt, row_amax, M, col_amax, K,
                                 st)) != NVFP4_OK)
            return s;
        return ok();
    }
    if (M == 0 || K == 0)
        return zero(row_amax, row_amax ? 1 : 0, col_amax, col_amax ? 1 : 0, st) != NVFP4_OK ? NVFP4_EDEVICE : ok();
    if ((s = amax_zero_first(AMAX_TENSOR, x, K, 0, M, nullptr, nullptr, row_amax, col_amax, gt, row_amax,
                             row_amax ? 1 : 0, col_amax, col_amax ? 1 : 0, st)) != NVFP4_OK)
        return s;
    return ok();
}

nvfp4_status nvfp4_encode(const void* xv, int64_t M, int64_t K, nvfp4_scaling mode,
                          const float* row_amax, const float* col_amax,
                          uint8_t* row_q, uint8_t* row_sf, uint8_t* col_q, uint8_t* col_sf, void* stream) {
    if (mode != NVFP4_PER_TENSOR && mode != NVFP4_PER_TOKEN)
        return fail(NVFP4_EINVAL, "nvfp4_encode takes PER_TENSOR or PER_TOKEN (mode %d)", (int)mode);
    Dir r = direction("row", row_q, row_sf, row_amax);
    if (r.st != NVFP4_OK) return r.st;
    Dir c = direction("col", col_q, col_sf, col_amax);
    if (c.st != NVFP4_OK) return c.st;
    if (!r.want && !c.want) return fail(NVFP4_EINVAL, "no output direction requested");
    nvfp4_status s = check_shape(M, K, r.want, c.want, mode);
    if (s != NVFP4_OK) return s;
    if (!xv) return fail(NVFP4_EINVAL, "x is NULL");
    if (!aligned(xv, 16)) return fail(NVFP4_EALIGN, "x must be 16-byte aligned");
    if (M == 0 || K == 0) return ok();
    const GroupTable gt = empty_table();
    if ((s = encode_launch([&](hipEvent_t b, hipEvent_t a) { return launch_encode(mode == NVFP4_PER_TOKEN ? ENC_TOKEN : ENC_TENSOR, r.want, c.want, true,
                                     static_cast<const uint16_t*>(xv), M, K, 0, M, row_amax, col_amax,
                                     row_q, row_sf, col_q, col_sf, nullptr, nullptr, gt, as_stream(stream), b, a); })) != NVFP4_OK)
        return s;
    return ok();
}

nvfp4_status nvfp4_quantize_grouped(const void* xv, int64_t K, int32_t num_groups, const int64_t* h_counts,
                                    uint8_t* row_q, uint8_t* row_sf, float* row_amax,
                                    uint8_t* col_q, uint8_t* col_sf, float* col_amax, void* stream) {
    if (num_groups < 0) return fail(NVFP4_EINVAL, "num_groups < 0");
    if (num_groups > 0 && !h_counts) return fail(NVFP4_EINVAL, "h_counts is NULL");
    Dir r = direction("row", row_q, row_sf, row_amax);
    if (r.st != NVFP4_OK) return r.st;
    Dir c = direction("col", col_q, col_sf, col_amax);
    if (c.st != NVFP4_OK) return c.st;
    if (!r.want && !c.want) return fail(NVFP4_EINVAL, "no output direction requested");
    int64_t T = 0;
    for (int32_t e = 0; e < num_groups; ++e) {
        if (h_counts[e] < 0 || h_counts[e] % 16 != 0)
            return fail(NVFP4_ESHAPE, "group %d has %lld rows; counts must be >= 0 and multiples of 16", e, (long long)h_counts[e]);
        T += h_counts[e];
    }
    nvfp4_status s = check_shape(T, K, r.want, c.want, NVFP4_PER_TOKEN);
    if (s != NVFP4_OK) return s;
    if (!xv && T > 0) return fail(NVFP4_EINVAL, "x is NULL");
    if (xv && !aligned(xv, 16)) return fail(NVFP4_EALIGN, "x must be 16-byte aligned");
    const uint16_t* x = static_cast<const uint16_t*>(xv);
    hipStream_t st = as_stream(stream);
    float* ra = r.want ? row_amax : nullptr;
    float* ca = c.want ? col_amax : nullptr;
    if (!c.want && T > 0 && K > 0 && rows_path(K)) {
        // rowwise only: per-token rowwise of all T rows, one read of x
        int cus = 0;
        if ((s = device_cus(st, &cus)) != NVFP4_OK) return s;
        const unsigned grid = rows_grid(cus, T, K);
        if ((s = encode_launch([&](hipEvent_t b, hipEvent_t a) {
                 return launch_rows(x, T, K, row_q, row_sf, ra, grid, st, b, a);
             })) != NVFP4_OK)
            return s;
        return ok();
    }
    // one amax launch (at most kMaxGroupsPerLaunch experts, or rowwise only)
    // zeroes its own outputs; several launches take a fill first
    const bool one_launch = !c.want || num_groups <= kMaxGroupsPerLaunch;
    if (T == 0 || K == 0 || !one_launch) {
        if ((s = zero(ra, T, ca, (int64_t)num_groups * K, st)) != NVFP4_OK) return s;
        if (T == 0 || K == 0) return ok();
    }
    if (!c.want) {
        const GroupTable gt = empty_table();
        if ((s = amax_zero_first(AMAX_TOKEN, x, K, 0, T, ra, nullptr, nullptr, nullptr, gt, ra, T, nullptr, 0, st)) != NVFP4_OK)
            return s;
        if ((s = encode_launch([&](hipEvent_t b, hipEvent_t a) { return launch_encode(ENC_TOKEN, true, false, false, x, T, K, 0, T, ra, nullptr, row_q, row_sf, nullptr, nullptr,
                                         nullptr, nullptr, gt, st, b, a); })) != NVFP4_OK) return s;
        return ok();
    }
    // experts travel in the kernel arguments, a bounded number per launch
    int64_t off = 0;
    for (int32_t e0 = 0; e0 < num_groups; e0 += kMaxGroupsPerLaunch) {
        GroupTable gt;
        gt.n = 0;
        gt.first = e0;
        const int64_t begin = off;
        for (int32_t e = e0; e < num_groups && e < e0 + kMaxGroupsPerLaunch; ++e) {
            gt.off[gt.n] = off;
            gt.cnt[gt.n] = h_counts[e];
            off += h_counts[e];
            ++gt.n;
        }
        const int64_t end = off;
        if (end == begin) continue;
        if (one_launch)
            s = amax_zero_first(AMAX_GROUPED, x, K, begin, end, ra, ca, nullptr, nullptr, gt, ra, T, ca,
                                (int64_t)num_groups * K, st);
        else
            s = check_hip(launch_amax(AMAX_GROUPED, x, K, begin, end, ra, ca, nullptr, nullptr, gt, st), "amax");
        if (s != NVFP4_OK) return s;
        if ((s = encode_launch([&](hipEvent_t b, hipEvent_t a) { return launch_encode(ENC_GROUPED, r.want, true, false, x, T, K, begin, end, ra, ca, row_q, row_sf, col_q, col_sf,
                                         nullptr, nullptr, gt, st, b, a); })) != NVFP4_OK) return s;
    }
    return ok();
}

nvfp4_status nvfp4_dequantize(const uint8_t* q, const uint8_t* sf, const float* amax, int64_t R, int64_t C,
                              nvfp4_scaling mode, int out_is_bf16, void* out, void* stream) {
    if (mode != NVFP4_PER_TENSOR && mode != NVFP4_PER_TOKEN && mode != NVFP4_TILE_16x16)
        return fail(NVFP4_EINVAL, "unknown scaling mode %d", (int)mode);
    if (R < 0 || C < 0) return fail(NVFP4_EINVAL, "negative size");
    if (C % 16 != 0) return fail(NVFP4_ESHAPE, "dequantize needs C %% 16 == 0 (C=%lld)", (long long)C);
    if (R == 0 || C == 0) return ok();
    if (!q || !sf || !amax || !out) return fail(NVFP4_EINVAL, "NULL argument");
    if (!aligned(q, 8) || !aligned(out, 16) || !aligned(amax, 4)) return fail(NVFP4_EALIGN, "q needs 8-byte, out 16-byte, amax 4-byte alignment");
    nvfp4_status s = check_hip(launch_dequant(q, sf, amax, R, C, mode == NVFP4_PER_TOKEN ? 1 : 0, out_is_bf16 != 0, out,
                                              as_stream(stream)), "dequantize");
    return s != NVFP4_OK ? s : ok();
}

namespace {

nvfp4_status gemm_impl(const uint8_t* a_q, const uint8_t* a_sf, const float* a_amax, int a_per_row,
                       const uint8_t* b_q, const uint8_t* b_sf, const float* b_amax, int b_per_row,
                       int64_t M, int64_t N, int64_t K, float* out, void* stream, bool swizzled) {
    if (M < 0 || N < 0 || K < 0) return fail(NVFP4_EINVAL, "negative size");
    if (K % 16 != 0) return fail(NVFP4_ESHAPE, "gemm needs K %% 16 == 0 (K=%lld)", (long long)K);
    if (K > kMaxGemmK) return fail(NVFP4_ESHAPE, "gemm needs K <= %lld (K=%lld)", (long long)kMaxGemmK, (long long)K);
    if (M > 0 && N > 0 && (M > kMaxGemmTiles || N > kMaxGemmTiles || ((M + 127) / 128) * ((N + 127) / 128) > kMaxGemmTiles))
        return fail(NVFP4_ESHAPE, "gemm needs cdiv(M, 128) * cdiv(N, 128) < 2^31 output tiles");
    if (M == 0 || N == 0) return ok();
    if (!out || !a_amax || !b_amax) return fail(NVFP4_EINVAL, "NULL argument");
    if (K > 0 && (!a_q || !a_sf || !b_q || !b_sf)) return fail(NVFP4_EINVAL, "NULL argument");
    if (!aligned(a_q, 16) || !aligned(b_q, 16)) return fail(NVFP4_EALIGN, "a_q and b_q must be 16-byte aligned");
    if (!aligned(a_amax, 4) || !aligned(b_amax, 4) || !aligned(out, 4))
        return fail(NVFP4_EALIGN, "amax and out must be 4-byte aligned");
    if (swizzled && (!aligned(a_sf, 4) || !aligned(b_sf, 4)))
        return fail(NVFP4_EALIGN, "swizzled scales must be 4-byte aligned");
    nvfp4_status s = encode_launch([&](hipEvent_t b, hipEvent_t a) {
        return launch_gemm_nvfp4(a_q, a_sf, a_amax, a_per_row ? 1 : 0, b_q, b_sf, b_amax, b_per_row ? 1 : 0, M, N, K,
                                 out, as_stream(stream), b, a, swizzled);
    });
    return s != NVFP4_OK ? s : ok();
}

}  // namespace

nvfp4_status nvfp4_gemm(const uint8_t* a_q, const uint8_t* a_sf, const float* a_amax, int a_per_row,
                        const uint8_t* b_q, const uint8_t* b_sf, const float* b_amax, int b_per_row,
                        int64_t M, int64_t N, int64_t K, float* out, void* stream) {
    return gemm_impl(a_q, a_sf, a_amax, a_per_row, b_q, b_sf, b_amax, b_per_row, M, N, K, out, stream, false);
}

nvfp4_status nvfp4_gemm_swizzled(const uint8_t* a_q, const uint8_t* a_sf, const float* a_amax, int a_per_row,
                                 const uint8_t* b_q, const uint8_t* b_sf, const float* b_amax, int b_per_row,
                                 int64_t M, int64_t N, int64_t K, float* out, void* stream) {
    return gemm_impl(a_q, a_sf, a_amax, a_per_row, b_q, b_sf, b_amax, b_per_row, M, N, K, out, stream, true);
}

nvfp4_status nvfp4_swizzle_scales(const uint8_t* sf, int64_t R, int64_t nb, uint8_t* out, void* stream) {
    if (R < 0 || nb < 0) return fail(NVFP4_EINVAL, "negative size");
    if (R > ((int64_t)1 << 40) || nb > ((int64_t)1 << 24)) return fail(NVFP4_ESHAPE, "scale matrix too large");
    if (R == 0 || nb == 0) return ok();
    if (!sf || !out) return fail(NVFP4_EINVAL, "NULL argument");
    if (!aligned(out, 4)) return fail(NVFP4_EALIGN, "out must be 4-byte aligned");
    nvfp4_status s = check_hip(launch_swizzle_scales(sf, R, nb, out, as_stream(stream)), "swizzle");
    return s != NVFP4_OK ? s : ok();
}

nvfp4_status nvfp4_gemm_grouped(const uint8_t* a_q, const uint8_t* a_sf, const float* a_amax, int a_per_row,
                                const uint8_t* b_q, const uint8_t* b_sf, const float* b_amax, int b_per_row,
                                int32_t num_groups, const int64_t* h_counts, int64_t N, int64_t K, float* out,
                                void* stream) {
    if (num_groups < 0 || N < 0 || K < 0) return fail(NVFP4_EINVAL, "negative size");
    if (num_groups > 0 && !h_counts) return fail(NVFP4_EINVAL, "h_counts is NULL");
    if (K % 16 != 0) return fail(NVFP4_ESHAPE, "gemm needs K %% 16 == 0 (K=%lld)", (long long)K);
    if (K > kMaxGemmK) return fail(NVFP4_ESHAPE, "gemm needs K <= %lld (K=%lld)", (long long)kMaxGemmK, (long long)K);
    int64_t T = 0, tiles = 0;
    for (int32_t e = 0; e < num_groups; ++e) {
        if (h_counts[e] < 0) return fail(NVFP4_ESHAPE, "group %d has a negative row count", e);
        if (h_counts[e] > kMaxGemmTiles || N > kMaxGemmTiles) return fail(NVFP4_ESHAPE, "group too large");
        T += h_counts[e];
        tiles += ((h_counts[e] + 127) / 128) * ((N + 127) / 128);
        if (tiles > kMaxGemmTiles) return fail(NVFP4_ESHAPE, "gemm needs fewer than 2^31 output tiles of 128 x 128");
    }
    if (T == 0 || N == 0) return ok();
    if (!out || !a_amax || !b_amax) return fail(NVFP4_EINVAL, "NULL argument");
    if (K > 0 && (!a_q || !a_sf || !b_q || !b_sf)) return fail(NVFP4_EINVAL, "NULL argument");
    if (!aligned(a_q, 16) || !aligned(b_q, 16)) return fail(NVFP4_EALIGN, "a_q and b_q must be 16-byte aligned");
    if (!aligned(a_amax, 4) || !aligned(b_amax, 4) || !aligned(out, 4))
        return fail(NVFP4_EALIGN, "amax and out must be 4-byte aligned");
    nvfp4_status s = encode_launch([&](hipEvent_t b, hipEvent_t a) {
        return launch_gemm_grouped(a_q, a_sf, a_amax, a_per_row ? 1 : 0, b_q, b_sf, b_amax, b_per_row ? 1 : 0,
                                   num_groups, h_counts, N, K, out, as_stream(stream), b, a);
    });
    return s != NVFP4_OK ? s : ok();
}

nvfp4_status nvfp4_amax_accumulate(float* buf, const float* observed, int64_t n, float decay, void* stream) {
    if (n < 0) return fail(NVFP4_EINVAL, "n < 0");
    if (!(decay >= 0.0f && decay <= 1.0f)) return fail(NVFP4_EINVAL, "decay must lie in [0, 1]");
    if (n == 0) return ok();
    if (!buf || !observed) return fail(NVFP4_EINVAL, "NULL argument");
    if (!aligned(buf, 4) || !aligned(observed, 4)) return fail(NVFP4_EALIGN, "buffers must be 4-byte aligned");
    nvfp4_status s = check_hip(launch_accumulate(buf, observed, n, decay, as_stream(stream)), "accumulate");
    return s != NVFP4_OK ? s : ok();
}

nvfp4_status nvfp4_amax_accumulate_reduce(float* buf, const float* observed, int64_t n, float decay, void* stream) {
    if (n < 0) return fail(NVFP4_EINVAL, "n < 0");
    if (!(decay >= 0.0f && decay <= 1.0f)) return fail(NVFP4_EINVAL, "decay must lie in [0, 1]");
    if (!buf || (n > 0 && !observed)) return fail(NVFP4_EINVAL, "NULL argument");
    if (!aligned(buf, 4) || (observed && !aligned(observed, 4))) return fail(NVFP4_EALIGN, "buffers must be 4-byte aligned");
    nvfp4_status s = check_hip(launch_accumulate_reduce(buf, observed, n, decay, as_stream(stream)), "accumulate");
    return s != NVFP4_OK ? s : ok();
}

}  // extern "C"
