// C-ABI of libkvmap: validation, the context (RoPE-table cache, workspace, scratch) and the
// launch sequence of each call.  Declarations and the contract of every entry point are in
// include/kvmap.h.

#include "../../include/kvmap.h"

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <new>
#include <vector>

#include "internal.h"

using namespace kvmap;

namespace {

thread_local std::string g_err;

int fail(int status, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return status;
}

int ok() {
    g_err.clear();
    return KVMAP_OK;
}

#define KVMAP_HIP(call)                                                                     \
    do {                                                                                    \
        hipError_t e_ = (call);                                                             \
        if (e_ != hipSuccess)                                                               \
            return fail(e_ == hipErrorOutOfMemory ? KVMAP_ERR_OUT_OF_MEMORY : KVMAP_ERR_DEVICE, \
                        "%s: %s (%s:%d)", #call, hipGetErrorString(e_), __FILE__, __LINE__); \
    } while (0)

// Makes the context's device current for the duration of a call.
struct DeviceGuard {
    int prev = -1;
    bool okay = false;
    explicit DeviceGuard(int dev) {
        if (hipGetDevice(&prev) != hipSuccess) prev = -1;
        okay = (hipSetDevice(dev) == hipSuccess);
    }
    ~DeviceGuard() {
        if (prev >= 0) (void)hipSetDevice(prev);
    }
};

constexpr int kMaxRopeTables = 8;
constexpr int kSelSlots = 8;
constexpr int kTimingRing = 128;

// HIP events of one KVMAP_FLAG_TIMING apply: before the RoPE tables, before the de-rotation,
// before the map GEMM, after it.  Created on the context's first timed apply.
struct TimingRec {
    hipEvent_t ev[4] = {};
    bool table_built = false;  // a RoPE table was built by that apply (else its table time is 0)
};

// One uploaded selection: layer_sel [L_tgt*k], the ascending list of the source layers it uses,
// and L_src as a sentinel.  `copied` is recorded right after the upload from `host`, so the
// staging buffer is reused only once that copy has run.
struct SelSlot {
    int32_t* dev = nullptr;
    int32_t* host = nullptr;  // pinned
    hipEvent_t copied = nullptr;
    bool pending = false;     // `copied` recorded and maybe not yet reached
    std::vector<int32_t> key;
    uint64_t last_use = 0;
};
constexpr int kGramMaxSplits = 64;

struct RopeEntry {
    double theta = 0;
    std::vector<double> freq;  // the model's own frequencies when given (then theta is unused)
    int64_t pos0 = 0;
    bool diff = false;  // recode table of (theta, pos0) -> (theta2, pos0_2)
    double theta2 = 0;
    std::vector<double> freq2;
    int64_t pos0_2 = 0;
    int d = 0;
    int64_t T_cap = 0;
    float2* tab = nullptr;
    uint64_t last_use = 0;
};

bool ranges_overlap(const void* a, size_t na, const void* b, size_t nb) {
    const char* pa = (const char*)a;
    const char* pb = (const char*)b;
    return pa < pb + nb && pb < pa + na;
}

}  // namespace

// ---------------------------------------------------------------------------------------
// The allocation-free statistics call's scratch: one file-scope device array per GPU, of a
// fixed size, held for as long as the library is loaded.  In host code `scratch` names a
// host-side stand-in, not device memory: the device address comes from hipGetSymbolAddress,
// resolved once per device with that device current (at kvmap_create) and kept per device.
// Every use on the device -- kernel arguments -- takes that resolved address, never the name.
// ---------------------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[KVMAP_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// The device address of `scratch` on `device`, which must be the current device.
int resolve_static_scratch(int device, void** out) {
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    *out = nullptr;
    if (device < 0 || device >= kMaxDevices)
        return fail(KVMAP_ERR_DEVICE, "static scratch: device %d beyond the %d the library tracks", device, kMaxDevices);
    if (!g_scratch_dev[device]) {
        void* ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(KVMAP_ERR_DEVICE, "static scratch: hipGetSymbolAddress on device %d: %s", device,
                        hipGetErrorString(e));
        g_scratch_dev[device] = ptr;
    }
    *out = g_scratch_dev[device];
    return KVMAP_OK;
}
}  // namespace

int kvmap::report(int status, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return status;
}

struct kvmap_ctx {
    int device = 0;
    int cus = 0;                  // compute units of the device (persistent launches)
    std::vector<RopeEntry> ropes;
    uint64_t clock = 0;
    void* ws = nullptr;
    size_t ws_bytes = 0;
    SelSlot sel[kSelSlots];       // uploaded selections (see upload_selection)
    size_t sel_cap = 0;           // int32 entries of every slot
    unsigned int* d_count = nullptr;
    int32_t* d_zero = nullptr;    // the one-entry layer list {0} of kvmap_recode
    void* ridge = nullptr;        // fp64 factor and right-hand sides of the device ridge solve
    RidgeOverlap ridge_ov{};      // side stream and events of the device ridge's lookahead
    size_t ridge_bytes = 0;
    float* gram = nullptr;
    size_t gram_floats = 0;
    uint16_t* gram_split = nullptr;  // bf16 co-moment operands of one sub-batch
    size_t gram_split_elems = 0;
    void* static_scratch = nullptr;  // this device's copy of `scratch` (kvmap_gram_noalloc)
    TimingRec timing[kTimingRing];  // events of the last kTimingRing KVMAP_FLAG_TIMING applies
    int64_t n_timed = 0;
};

int kvmap::context_device(const kvmap_ctx* c) { return c ? c->device : -1; }

// ---------------------------------------------------------------------------------------
// status / version
// ---------------------------------------------------------------------------------------

extern "C" const char* kvmap_status_string(int status) {
    switch (status) {
        case KVMAP_OK: return "KVMAP_OK";
        case KVMAP_ERR_INVALID_ARGUMENT: return "KVMAP_ERR_INVALID_ARGUMENT";
        case KVMAP_ERR_SHAPE: return "KVMAP_ERR_SHAPE";
        case KVMAP_ERR_UNSUPPORTED: return "KVMAP_ERR_UNSUPPORTED";
        case KVMAP_ERR_NONFINITE: return "KVMAP_ERR_NONFINITE";
        case KVMAP_ERR_NOT_SPD: return "KVMAP_ERR_NOT_SPD";
        case KVMAP_ERR_DEVICE: return "KVMAP_ERR_DEVICE";
        case KVMAP_ERR_OUT_OF_MEMORY: return "KVMAP_ERR_OUT_OF_MEMORY";
        default: return "KVMAP_ERR_UNKNOWN";
    }
}

extern "C" const char* kvmap_last_error(void) { return g_err.c_str(); }

extern "C" int kvmap_version(void) { return KVMAP_VERSION; }

// ---------------------------------------------------------------------------------------
// context
// ---------------------------------------------------------------------------------------

extern "C" int kvmap_create(kvmap_ctx** out, int device) {
    if (!out) return fail(KVMAP_ERR_INVALID_ARGUMENT, "kvmap_create: out is NULL");
    *out = nullptr;
    int n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess || n <= 0)
        return fail(KVMAP_ERR_DEVICE, "kvmap_create: no HIP device visible");
    if (device < 0 || device >= n)
        return fail(KVMAP_ERR_DEVICE, "kvmap_create: device %d out of range [0, %d)", device, n);
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, device) != hipSuccess)
        return fail(KVMAP_ERR_DEVICE, "kvmap_create: cannot query device %d", device);
    if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
        return fail(KVMAP_ERR_DEVICE, "kvmap_create: device %d is %s, the kernels are built for gfx950",
                    device, prop.gcnArchName);
    DeviceGuard g(device);
    if (!g.okay) return fail(KVMAP_ERR_DEVICE, "kvmap_create: hipSetDevice(%d) failed", device);
    kvmap_ctx* c = new kvmap_ctx();
    c->device = device;
    c->cus = prop.multiProcessorCount;
    {
        const int r = resolve_static_scratch(device, &c->static_scratch);
        if (r) {
            const std::string msg = g_err;
            kvmap_destroy(c);
            return fail(r, "kvmap_create: %s", msg.c_str());
        }
    }
    const int32_t zero = 0;
    if (hipMalloc((void**)&c->d_count, sizeof(unsigned int)) != hipSuccess ||
        hipMalloc((void**)&c->d_zero, sizeof(int32_t)) != hipSuccess) {
        kvmap_destroy(c);
        return fail(KVMAP_ERR_OUT_OF_MEMORY, "kvmap_create: hipMalloc failed");
    }
    if (hipMemcpy(c->d_zero, &zero, sizeof zero, hipMemcpyHostToDevice) != hipSuccess) {
        kvmap_destroy(c);
        return fail(KVMAP_ERR_DEVICE, "kvmap_create: hipMemcpy failed");
    }
    *out = c;
    return ok();
}

extern "C" int kvmap_destroy(kvmap_ctx* c) {
    if (!c) return ok();
    DeviceGuard g(c->device);
    (void)hipDeviceSynchronize();
    for (auto& r : c->ropes) (void)hipFree(r.tab);
    (void)hipFree(c->ws);
    for (auto& sl : c->sel) {
        (void)hipFree(sl.dev);
        (void)hipHostFree(sl.host);
        if (sl.copied) (void)hipEventDestroy(sl.copied);
    }
    (void)hipFree(c->d_count);
    (void)hipFree(c->d_zero);
    (void)hipFree(c->ridge);
    if (c->ridge_ov.side) (void)hipStreamDestroy(c->ridge_ov.side);
    if (c->ridge_ov.main_ready) (void)hipEventDestroy(c->ridge_ov.main_ready);
    if (c->ridge_ov.side_done) (void)hipEventDestroy(c->ridge_ov.side_done);
    if (c->ridge_ov.side_done2) (void)hipEventDestroy(c->ridge_ov.side_done2);
    if (c->ridge_ov.fwd) (void)hipStreamDestroy(c->ridge_ov.fwd);
    if (c->ridge_ov.fwd_ready) (void)hipEventDestroy(c->ridge_ov.fwd_ready);
    if (c->ridge_ov.fwd_done) (void)hipEventDestroy(c->ridge_ov.fwd_done);
    (void)hipFree(c->gram);
    (void)hipFree(c->gram_split);
    for (auto& r : c->timing)
        for (auto& e : r.ev)
            if (e) (void)hipEventDestroy(e);
    delete c;
    return ok();
}

// ---------------------------------------------------------------------------------------
// validation
// ---------------------------------------------------------------------------------------

// d: the head dim, already validated (64 or 128); inv_freq, if given, has d/2 entries.
static int validate_rope(const kvmap_rope* r, const char* which, int64_t T, int d) {
    if (!r) return fail(KVMAP_ERR_INVALID_ARGUMENT, "%s RoPE descriptor is NULL", which);
    if (r->style != KVMAP_ROPE_HALF_SPLIT)
        return fail(KVMAP_ERR_UNSUPPORTED, "%s RoPE style %d refused: only the half-split form is mapped",
                    which, (int)r->style);
    if (r->inv_freq) {
        for (int i = 0; i < d / 2; ++i)
            if (!(r->inv_freq[i] >= 0.0) || !std::isfinite(r->inv_freq[i]))
                return fail(KVMAP_ERR_INVALID_ARGUMENT, "%s RoPE inv_freq[%d] must be finite and >= 0", which, i);
    } else if (!(r->theta > 0.0) || !std::isfinite(r->theta)) {
        return fail(KVMAP_ERR_INVALID_ARGUMENT, "%s RoPE theta must be finite and > 0", which);
    }
    if (r->pos0 < 0) return fail(KVMAP_ERR_INVALID_ARGUMENT, "%s RoPE pos0 must be >= 0", which);
    if (r->pos0 > (int64_t(1) << 31) - T)
        return fail(KVMAP_ERR_INVALID_ARGUMENT, "%s RoPE pos0 + T exceeds 2^31", which);
    return KVMAP_OK;
}

// The shape and dtype checks of an apply call (everything but layer_sel and the RoPE
// descriptors): shared by kvmap_validate_apply and kvmap_reserve.
static int validate_dims(const kvmap_dims* d) {
    if (!d) return fail(KVMAP_ERR_INVALID_ARGUMENT, "dims is NULL");
    if (d->dtype != KVMAP_DTYPE_BF16 && d->dtype != KVMAP_DTYPE_F32)
        return fail(KVMAP_ERR_UNSUPPORTED, "dtype %d unknown", (int)d->dtype);
    if (d->L_src < 1 || d->L_tgt < 1 || d->H_kv < 1 || d->k < 1)
        return fail(KVMAP_ERR_SHAPE, "L_src, L_tgt, H_kv and k must be >= 1");
    if (d->T < 1) return fail(KVMAP_ERR_SHAPE, "T must be >= 1");
    if (d->head_dim < 2 || (d->head_dim & 1))
        return fail(KVMAP_ERR_SHAPE, "head_dim %d must be even", (int)d->head_dim);
    if (d->head_dim != 64 && d->head_dim != 128)
        return fail(KVMAP_ERR_UNSUPPORTED, "head_dim %d: only 64 and 128 are built", (int)d->head_dim);
    if (d->k > d->L_src) return fail(KVMAP_ERR_SHAPE, "k=%d exceeds L_src=%d", (int)d->k, (int)d->L_src);
    if (d->k > 64) return fail(KVMAP_ERR_UNSUPPORTED, "k=%d: at most 64 selected layers are built", (int)d->k);
    const int64_t N = (int64_t)d->H_kv * d->head_dim;
    const int64_t F = N * d->k;
    if (N * F >= (int64_t(1) << 31))
        return fail(KVMAP_ERR_SHAPE, "one target layer's map (N*F = %lld) must stay below 2^31 entries",
                    (long long)(N * F));
    if (d->T * d->head_dim >= (int64_t(1) << 31))
        return fail(KVMAP_ERR_SHAPE, "T*head_dim must stay below 2^31");
    if ((int64_t)d->L_tgt * d->k >= (int64_t(1) << 24))
        return fail(KVMAP_ERR_SHAPE, "L_tgt*k too large");
    return KVMAP_OK;
}

extern "C" int kvmap_validate_apply(const kvmap_dims* d, const int32_t* layer_sel,
                                    const kvmap_rope* rs, const kvmap_rope* rt) {
    int st = validate_dims(d);
    if (st) return st;
    if (!layer_sel) return fail(KVMAP_ERR_INVALID_ARGUMENT, "layer_sel is NULL");
    st = validate_rope(rs, "source", d->T, d->head_dim);
    if (st) return st;
    st = validate_rope(rt, "target", d->T, d->head_dim);
    if (st) return st;
    std::vector<char> seen(d->L_src, 0);
    for (int t = 0; t < d->L_tgt; ++t) {
        for (int j = 0; j < d->k; ++j) {
            const int32_t s = layer_sel[(size_t)t * d->k + j];
            if (s < 0 || s >= d->L_src)
                return fail(KVMAP_ERR_SHAPE, "layer_sel[%d][%d] = %d outside [0, %d)", t, j, (int)s, (int)d->L_src);
            if (seen[s])
                return fail(KVMAP_ERR_SHAPE, "layer_sel[%d] selects source layer %d twice", t, (int)s);
            seen[s] = 1;
        }
        for (int j = 0; j < d->k; ++j) seen[layer_sel[(size_t)t * d->k + j]] = 0;
    }
    return ok();
}

// ---------------------------------------------------------------------------------------
// apply
// ---------------------------------------------------------------------------------------

// Cached fp32 tables built in fp64: a RoPE table of r, or (r2 given) the recode table
// from r to r2.
static bool same_freqs(double theta, const std::vector<double>& f, const kvmap_rope* r, int d) {
    if (r->inv_freq) return (int)f.size() == d / 2 && std::equal(f.begin(), f.end(), r->inv_freq);
    return f.empty() && theta == r->theta;
}

static RopeFreqs make_freqs(const kvmap_rope* r, int d) {
    RopeFreqs fr{};
    fr.theta = r->theta;
    fr.given = r->inv_freq != nullptr;
    for (int i = 0; fr.given && i < d / 2; ++i) fr.f[i] = r->inv_freq[i];
    return fr;
}

static std::vector<double> freq_list(const kvmap_rope* r, int d) {
    return r->inv_freq ? std::vector<double>(r->inv_freq, r->inv_freq + d / 2) : std::vector<double>();
}

static int get_rope_table(kvmap_ctx* c, const kvmap_rope* r, int d, int64_t T, hipStream_t s,
                          float2** out, bool* built, const kvmap_rope* r2 = nullptr) {
    *built = false;
    const bool diff = r2 != nullptr;
    for (auto& e : c->ropes) {
        if (same_freqs(e.theta, e.freq, r, d) && e.pos0 == r->pos0 && e.d == d && e.T_cap >= T && e.diff == diff &&
            (!diff || (same_freqs(e.theta2, e.freq2, r2, d) && e.pos0_2 == r2->pos0))) {
            e.last_use = ++c->clock;
            *out = e.tab;
            return KVMAP_OK;
        }
    }
    if ((int)c->ropes.size() >= kMaxRopeTables) {
        // Evict the least recently used table once no queued work can still read it.
        KVMAP_HIP(hipDeviceSynchronize());
        auto it = std::min_element(c->ropes.begin(), c->ropes.end(),
                                   [](const RopeEntry& a, const RopeEntry& b) { return a.last_use < b.last_use; });
        (void)hipFree(it->tab);
        c->ropes.erase(it);
    }
    RopeEntry e;
    e.theta = r->theta;
    e.freq = freq_list(r, d);
    e.pos0 = r->pos0;
    e.diff = diff;
    e.theta2 = diff ? r2->theta : 0.0;
    if (diff) e.freq2 = freq_list(r2, d);
    e.pos0_2 = diff ? r2->pos0 : 0;
    e.d = d;
    e.T_cap = T;
    KVMAP_HIP(hipMalloc((void**)&e.tab, (size_t)T * (d / 2) * sizeof(float2)));
    hipError_t err = diff ? launch_rope_diff_table(e.tab, T, d, make_freqs(r, d), r->pos0, make_freqs(r2, d), r2->pos0, s)
                          : launch_rope_table(e.tab, T, d, make_freqs(r, d), r->pos0, s);
    if (err != hipSuccess) {
        (void)hipFree(e.tab);
        return fail(KVMAP_ERR_DEVICE, "RoPE table launch: %s", hipGetErrorString(err));
    }
    e.last_use = ++c->clock;
    c->ropes.push_back(e);
    *out = e.tab;
    *built = true;
    return KVMAP_OK;
}

// Every slot holds `entries` int32 entries; growing them waits for the device (queued kernels
// may still read the old buffers), like the workspace's growth.
static int ensure_sel_slots(kvmap_ctx* c, size_t entries) {
    if (entries <= c->sel_cap) return KVMAP_OK;
    KVMAP_HIP(hipDeviceSynchronize());
    for (auto& sl : c->sel) {
        (void)hipFree(sl.dev);
        (void)hipHostFree(sl.host);
        sl.dev = nullptr;
        sl.host = nullptr;
        sl.key.clear();
        sl.pending = false;
    }
    c->sel_cap = 0;
    for (auto& sl : c->sel) {
        if (!sl.copied) KVMAP_HIP(hipEventCreateWithFlags(&sl.copied, hipEventDisableTiming));
        KVMAP_HIP(hipMalloc((void**)&sl.dev, entries * sizeof(int32_t)));
        KVMAP_HIP(hipHostMalloc((void**)&sl.host, entries * sizeof(int32_t), hipHostMallocDefault));
    }
    c->sel_cap = entries;
    return KVMAP_OK;
}

static size_t sel_entries(const kvmap_dims* d) { return (size_t)d->L_tgt * d->k + d->L_src + 1; }

// The device copy of layer_sel plus the ascending list of the source layers it uses.  A
// selection already held by a slot is reused as is; a new one goes to the least recently used
// slot through its pinned staging buffer with an asynchronous copy on `s`, so the host never
// waits for the stream -- unless that slot's previous upload has not run yet, i.e. the caller has
// queued kSelSlots applies with other selections behind it.  Queued kernels that still read an
// overwritten slot are ordered before the copy by the stream (calls sharing a context share
// one stream, or the caller orders them).
static int upload_selection(kvmap_ctx* c, const kvmap_dims* d, const int32_t* layer_sel, hipStream_t s,
                            int* n_used, const int32_t** dev) {
    const size_t nsel = (size_t)d->L_tgt * d->k;
    std::vector<int32_t> want(layer_sel, layer_sel + nsel);
    std::vector<char> used(d->L_src, 0);
    for (size_t i = 0; i < nsel; ++i) used[want[i]] = 1;
    for (int l = 0; l < d->L_src; ++l)
        if (used[l]) want.push_back(l);
    *n_used = (int)(want.size() - nsel);
    want.push_back(d->L_src);  // sentinel: distinguishes equal selections over different L_src
    int st = ensure_sel_slots(c, sel_entries(d));
    if (st) return st;
    SelSlot* slot = nullptr;
    for (auto& sl : c->sel)
        if (sl.key == want) slot = &sl;
    if (!slot) {
        slot = &c->sel[0];
        for (auto& sl : c->sel)
            if (sl.last_use < slot->last_use) slot = &sl;
        if (slot->pending) {
            KVMAP_HIP(hipEventSynchronize(slot->copied));  // the staging buffer's last copy
            slot->pending = false;
        }
        slot->key.clear();  // invalid until the copy below is queued
        memcpy(slot->host, want.data(), want.size() * sizeof(int32_t));
        KVMAP_HIP(hipMemcpyAsync(slot->dev, slot->host, want.size() * sizeof(int32_t), hipMemcpyHostToDevice, s));
        KVMAP_HIP(hipEventRecord(slot->copied, s));
        slot->pending = true;
        slot->key = want;
    }
    slot->last_use = ++c->clock;
    *dev = slot->dev;
    return KVMAP_OK;
}

static int ensure_workspace(kvmap_ctx* c, size_t bytes) {
    if (bytes <= c->ws_bytes) return KVMAP_OK;
    KVMAP_HIP(hipDeviceSynchronize());
    (void)hipFree(c->ws);
    c->ws = nullptr;
    c->ws_bytes = 0;
    KVMAP_HIP(hipMalloc(&c->ws, bytes));
    c->ws_bytes = bytes;
    return KVMAP_OK;
}

// De-rotated source keys, then (short bf16 caches) the short-cache kernel's fp32 partial sums.
static size_t derope_bytes(const kvmap_dims* d) {
    const size_t es = d->dtype == KVMAP_DTYPE_BF16 ? 2 : 4;
    return ((size_t)d->L_src * d->H_kv * (size_t)d->T * d->head_dim * es + 255) & ~(size_t)255;
}

static bool small_path(const kvmap_dims* d) { return d->dtype == KVMAP_DTYPE_BF16 && d->T <= kSmallT; }

static size_t workspace_bytes(const kvmap_ctx* c, const kvmap_dims* d) {
    size_t b = derope_bytes(d);
    if (small_path(d)) {
        const ApplyGeom g{d->L_src, d->L_tgt, d->H_kv, d->head_dim, d->k, d->T};
        b += map_bf16_small_plan(g, c->cus).part_bytes;
    }
    return b;
}

extern "C" int kvmap_reserve(kvmap_ctx* c, const kvmap_dims* d) {
    // the dims first: a refused shape never reaches the workspace arithmetic
    int st = validate_dims(d);
    if (st) return st;
    if (!c) return fail(KVMAP_ERR_INVALID_ARGUMENT, "kvmap_reserve: ctx is NULL");
    DeviceGuard g(c->device);
    st = ensure_workspace(c, workspace_bytes(c, d));
    if (st) return st;
    st = ensure_sel_slots(c, sel_entries(d));
    if (st) return st;
    return ok();
}

extern "C" int kvmap_validate_apply_buffers(const kvmap_dims* d, const void* src_k, const void* src_v,
                                            const void* W_k, const void* b_k, const void* W_v, const void* b_v,
                                            const void* tgt_k, const void* tgt_v) {
    int st = validate_dims(d);
    if (st) return st;
    if (!src_k || !src_v || !W_k || !b_k || !W_v || !b_v || !tgt_k || !tgt_v)
        return fail(KVMAP_ERR_INVALID_ARGUMENT, "kvmap_apply: NULL device pointer");
    const void* ptrs[8] = {src_k, src_v, W_k, b_k, W_v, b_v, tgt_k, tgt_v};
    for (const void* p : ptrs)
        if (((uintptr_t)p) & 15) return fail(KVMAP_ERR_INVALID_ARGUMENT, "kvmap_apply: pointers must be 16-byte aligned");
    const ApplyGeom g{d->L_src, d->L_tgt, d->H_kv, d->head_dim, d->k, d->T};
    const size_t es = d->dtype == KVMAP_DTYPE_BF16 ? 2 : 4;
    const size_t src_bytes = (size_t)g.L_src * g.H * g.T * g.d * es;
    const size_t tgt_bytes = (size_t)g.L_tgt * g.H * g.T * g.d * es;
    const size_t w_bytes = (size_t)g.L_tgt * g.N() * g.F() * es;
    const size_t b_bytes = (size_t)g.L_tgt * g.N() * es;
    const void* ins[6] = {src_k, src_v, W_k, b_k, W_v, b_v};
    const size_t insz[6] = {src_bytes, src_bytes, w_bytes, b_bytes, w_bytes, b_bytes};
    for (int i = 0; i < 6; ++i)
        if (ranges_overlap(ins[i], insz[i], tgt_k, tgt_bytes) || ranges_overlap(ins[i], insz[i], tgt_v, tgt_bytes))
            return fail(KVMAP_ERR_INVALID_ARGUMENT, "kvmap_apply: an input overlaps an output");
    if (ranges_overlap(tgt_k, tgt_bytes, tgt_v, tgt_bytes))
        return fail(KVMAP_ERR_INVALID_ARGUMENT, "kvmap_apply: tgt_k and tgt_v overlap");
    return ok();
}

extern "C" int kvmap_apply(kvmap_ctx* c, const kvmap_dims* d, const void* src_k, const void* src_v,
                           const int32_t* layer_sel, const void* W_k, const void* b_k, const void* W_v,
                           const void* b_v, const kvmap_rope* rope_src, const kvmap_rope* rope_tgt,
                           void* tgt_k, void* tgt_v, void* stream, uint32_t flags) {
    if (!c) return fail(KVMAP_ERR_INVALID_ARGUMENT, "kvmap_apply: ctx is NULL");
    int st = kvmap_validate_apply(d, layer_sel, rope_src, rope_tgt);
    if (st) return st;
    st = kvmap_validate_apply_buffers(d, src_k, src_v, W_k, b_k, W_v, b_v, tgt_k, tgt_v);
    if (st) return st;
    if (flags & ~(KVMAP_FLAG_CHECK_FINITE | KVMAP_FLAG_TIMING))
        return fail(KVMAP_ERR_INVALID_ARGUMENT, "kvmap_apply: unknown flag bits 0x%x", flags);
    const ApplyGeom g{d->L_src, d->L_tgt, d->H_kv, d->head_dim, d->k, d->T};

    DeviceGuard guard(c->device);
    if (!guard.okay) return fail(KVMAP_ERR_DEVICE, "kvmap_apply: hipSetDevice(%d) failed", c->device);
    hipStream_t s = (hipStream_t)stream;
    const bool timing = (flags & KVMAP_FLAG_TIMING) != 0;
    TimingRec& tr = c->timing[c->n_timed % kTimingRing];
    if (timing && !tr.ev[0]) {
        for (auto& r : c->timing)
            for (auto& e : r.ev) KVMAP_HIP(hipEventCreate(&e));
    }

    if (timing) KVMAP_HIP(hipEventRecord(tr.ev[0], s));
    float2 *tab_src = nullptr, *tab_tgt = nullptr;
    bool b1 = false, b2 = false;
    st = get_rope_table(c, rope_src, g.d, g.T, s, &tab_src, &b1);
    if (st) return st;
    st = get_rope_table(c, rope_tgt, g.d, g.T, s, &tab_tgt, &b2);
    if (st) return st;
    int n_used = 0;
    const int32_t* d_sel = nullptr;
    st = upload_selection(c, d, layer_sel, s, &n_used, &d_sel);
    if (st) return st;
    st = ensure_workspace(c, workspace_bytes(c, d));
    if (st) return st;

    const Elem e = d->dtype == KVMAP_DTYPE_BF16 ? Elem::BF16 : Elem::F32;
    if (timing) KVMAP_HIP(hipEventRecord(tr.ev[1], s));
    KVMAP_HIP(launch_derope(e, src_k, c->ws, d_sel + (size_t)g.L_tgt * g.k, n_used, g, tab_src, s));
    if (timing) KVMAP_HIP(hipEventRecord(tr.ev[2], s));
    MapArgs a{c->ws, src_v, d_sel, W_k, b_k, W_v, b_v, tab_tgt, tgt_k, tgt_v};
    if (small_path(d))
        KVMAP_HIP(launch_map_bf16_small(a, g, map_bf16_small_plan(g, c->cus), (float*)((char*)c->ws + derope_bytes(d)), s));
    else if (e == Elem::BF16)
        KVMAP_HIP(launch_map_bf16(a, g, c->cus, s));
    else
        KVMAP_HIP(launch_map_f32(a, g, s));
    if (timing) {
        KVMAP_HIP(hipEventRecord(tr.ev[3], s));
        tr.table_built = b1 || b2;
        ++c->n_timed;
    }

    if (flags & KVMAP_FLAG_CHECK_FINITE) {
        const int64_t n = (int64_t)g.L_tgt * g.H * g.T * g.d;
        KVMAP_HIP(launch_fill_zero((float*)c->d_count, 1, s));  // a kernel, not a memset node
        KVMAP_HIP(launch_count_nonfinite(e, tgt_k, n, c->d_count, s));
        KVMAP_HIP(launch_count_nonfinite(e, tgt_v, n, c->d_count, s));
        unsigned int h = 0;
        KVMAP_HIP(hipMemcpyAsync(&h, c->d_count, sizeof h, hipMemcpyDeviceToHost, s));
        KVMAP_HIP(hipStreamSynchronize(s));
        if (h) return fail(KVMAP_ERR_NONFINITE, "kvmap_apply: %u non-finite values in the mapped cache", h);
    }
    return ok();
}

// ---------------------------------------------------------------------------------------
// RoPE recode (identity map: one rotation per pair)
// ---------------------------------------------------------------------------------------

extern "C" int kvmap_recode(kvmap_ctx* c, int32_t rows, int64_t T, int32_t head_dim, int32_t dtype,
                            const void* src, void* dst, const kvmap_rope* rope_src, const kvmap_rope* rope_tgt,
                            void* stream) {
    if (!c) return fail(KVMAP_ERR_INVALID_ARGUMENT, "kvmap_recode: ctx is NULL");
    if (rows < 1 || T < 1 || T > (int64_t(1) << 31) || (int64_t)rows * T > (int64_t(1) << 40))
        return fail(KVMAP_ERR_SHAPE, "kvmap_recode: rows=%d, T=%lld out of range", (int)rows, (long long)T);
    if (dtype != KVMAP_DTYPE_BF16 && dtype != KVMAP_DTYPE_F32)
        return fail(KVMAP_ERR_UNSUPPORTED, "kvmap_recode: dtype %d unknown", (int)dtype);
    if (head_dim != 64 && head_dim != 128)
        return fail(KVMAP_ERR_UNSUPPORTED, "kvmap_recode: head_dim %d (64 or 128 supported)", (int)head_dim);
    int st = validate_rope(rope_src, "source", T, head_dim);
    if (st) return st;
    st = validate_rope(rope_tgt, "target", T, head_dim);
    if (st) return st;
    if (!src || !dst) return fail(KVMAP_ERR_INVALID_ARGUMENT, "kvmap_recode: NULL device pointer");
    if ((((uintptr_t)src) | ((uintptr_t)dst)) & 15)
        return fail(KVMAP_ERR_INVALID_ARGUMENT, "kvmap_recode: pointers must be 16-byte aligned");
    const size_t es = dtype == KVMAP_DTYPE_BF16 ? 2 : 4;
    const size_t bytes = (size_t)rows * (size_t)T * head_dim * es;
    if (ranges_overlap(src, bytes, dst, bytes)) return fail(KVMAP_ERR_INVALID_ARGUMENT, "kvmap_recode: src and dst overlap");
    DeviceGuard guard(c->device);
    if (!guard.okay) return fail(KVMAP_ERR_DEVICE, "kvmap_recode: hipSetDevice(%d) failed", c->device);
    hipStream_t s = (hipStream_t)stream;
    float2* tab = nullptr;
    bool built = false;
    st = get_rope_table(c, rope_src, head_dim, T, s, &tab, &built, rope_tgt);
    if (st) return st;
    // all rows as the heads of one layer, listed by the single entry {0}
    const ApplyGeom g{1, 1, rows, head_dim, 1, T};
    const Elem e = dtype == KVMAP_DTYPE_BF16 ? Elem::BF16 : Elem::F32;
    KVMAP_HIP(launch_derope(e, src, dst, c->d_zero, 1, g, tab, s));
    return ok();
}

// ---------------------------------------------------------------------------------------
// fit-side rows from calibration caches
// ---------------------------------------------------------------------------------------

extern "C" int kvmap_cache_rows(kvmap_ctx* c, const void* cache, int32_t L, int32_t H, int64_t T, int32_t head_dim,
                                int32_t dtype, const int32_t* layers, int32_t n_layers, const kvmap_rope* rope,
                                void* out, void* stream) {
    if (!c) return fail(KVMAP_ERR_INVALID_ARGUMENT, "kvmap_cache_rows: ctx is NULL");
    if (L < 1 || H < 1 || T < 1 || T > (int64_t(1) << 31))
        return fail(KVMAP_ERR_SHAPE, "kvmap_cache_rows: L=%d, H=%d, T=%lld out of range", (int)L, (int)H, (long long)T);
    if (head_dim != 64 && head_dim != 128)
        return fail(KVMAP_ERR_UNSUPPORTED, "kvmap_cache_rows: head_dim %d (64 or 128 supported)", (int)head_dim);
    if (dtype != KVMAP_DTYPE_BF16 && dtype != KVMAP_DTYPE_F32)
        return fail(KVMAP_ERR_UNSUPPORTED, "kvmap_cache_rows: dtype %d unknown", (int)dtype);
    if (!layers || n_layers < 1 || n_layers > kMaxRowLayers)
        return fail(KVMAP_ERR_SHAPE, "kvmap_cache_rows: n_layers must be in [1, %d]", kMaxRowLayers);
    RowLayers rl{};
    for (int j = 0; j < n_layers; ++j) {
        if (layers[j] < 0 || layers[j] >= L)
            return fail(KVMAP_ERR_SHAPE, "kvmap_cache_rows: layers[%d] = %d outside [0, %d)", j, (int)layers[j], (int)L);
        rl.l[j] = layers[j];
    }
    if (rope) {
        int st = validate_rope(rope, "rows", T, head_dim);
        if (st) return st;
    }
    if (!cache || !out) return fail(KVMAP_ERR_INVALID_ARGUMENT, "kvmap_cache_rows: NULL device pointer");
    if ((((uintptr_t)cache) | ((uintptr_t)out)) & 15)
        return fail(KVMAP_ERR_INVALID_ARGUMENT, "kvmap_cache_rows: pointers must be 16-byte aligned");
    const size_t es = dtype == KVMAP_DTYPE_BF16 ? 2 : 4;
    const size_t in_bytes = (size_t)L * H * (size_t)T * head_dim * es;
    const size_t out_bytes = (size_t)n_layers * H * (size_t)T * head_dim * es;
    if (ranges_overlap(cache, in_bytes, out, out_bytes))
        return fail(KVMAP_ERR_INVALID_ARGUMENT, "kvmap_cache_rows: out overlaps the cache");
    DeviceGuard guard(c->device);
    if (!guard.okay) return fail(KVMAP_ERR_DEVICE, "kvmap_cache_rows: hipSetDevice(%d) failed", c->device);
    hipStream_t s = (hipStream_t)stream;
    float2* tab = nullptr;
    if (rope) {
        bool built = false;
        int st = get_rope_table(c, rope, head_dim, T, s, &tab, &built);
        if (st) return st;
    }
    const Elem e = dtype == KVMAP_DTYPE_BF16 ? Elem::BF16 : Elem::F32;
    KVMAP_HIP(launch_rows(e, cache, out, rl, n_layers, H, T, head_dim, tab, s));
    return ok();
}

extern "C" int kvmap_timings(kvmap_ctx* c, int32_t back, float* ms, int n_ms) {
    if (!c || !ms || n_ms < 3) return fail(KVMAP_ERR_INVALID_ARGUMENT, "kvmap_timings: bad arguments");
    const int64_t held = std::min<int64_t>(c->n_timed, kTimingRing);
    if (back < 0 || back >= held)
        return fail(KVMAP_ERR_INVALID_ARGUMENT, "kvmap_timings: %d timed applies held, asked for number %d back",
                    (int)held, (int)back);
    DeviceGuard g(c->device);
    const TimingRec& tr = c->timing[(c->n_timed - 1 - back) % kTimingRing];
    KVMAP_HIP(hipEventSynchronize(tr.ev[3]));
    float t01 = 0, t12 = 0, t23 = 0;
    KVMAP_HIP(hipEventElapsedTime(&t01, tr.ev[0], tr.ev[1]));
    KVMAP_HIP(hipEventElapsedTime(&t12, tr.ev[1], tr.ev[2]));
    KVMAP_HIP(hipEventElapsedTime(&t23, tr.ev[2], tr.ev[3]));
    ms[0] = tr.table_built ? t01 : 0.f;
    ms[1] = t12;
    ms[2] = t23;
    return ok();
}

extern "C" int kvmap_last_timings(kvmap_ctx* c, float* ms, int n_ms) {
    if (c && c->n_timed == 0) return fail(KVMAP_ERR_INVALID_ARGUMENT, "kvmap_last_timings: no timed apply recorded");
    return kvmap_timings(c, 0, ms, n_ms);
}

// ---------------------------------------------------------------------------------------
// fit-side statistics
// ---------------------------------------------------------------------------------------

static int validate_state(const kvmap_gram_state* st, const char* which) {
    if (!st) return fail(KVMAP_ERR_INVALID_ARGUMENT, "%s state is NULL", which);
    if (st->p < 4 || st->q < 4 || (st->p & 3) || (st->q & 3) || st->p > 65536 || st->q > 65536)
        return fail(KVMAP_ERR_SHAPE, "%s state: p=%d, q=%d must be multiples of 4 in [4, 65536]", which,
                    (int)st->p, (int)st->q);
    if (st->n < 0) return fail(KVMAP_ERR_SHAPE, "%s state: n < 0", which);
    if (st->xx_block < 0 || (st->xx_block && ((st->xx_block & 3) || st->p % st->xx_block)))
        return fail(KVMAP_ERR_SHAPE, "%s state: xx_block=%d must be 0 or a multiple of 4 dividing p=%d", which,
                    (int)st->xx_block, (int)st->p);
    if (!st->mean_x || !st->mean_y || !st->M_xx || !st->M_xy)
        return fail(KVMAP_ERR_INVALID_ARGUMENT, "%s state: NULL array", which);
    const void* arr[5] = {st->mean_x, st->mean_y, st->M_xx, st->M_xy, st->ss_y};
    for (const void* a : arr)
        if (((uintptr_t)a) & 15) return fail(KVMAP_ERR_INVALID_ARGUMENT, "%s state: arrays must be 16-byte aligned", which);
    return KVMAP_OK;
}

static int ensure_gram_scratch(kvmap_ctx* c, int p, int q, int64_t split_rows) {
    const size_t need = gram_scratch_floats(p, q, kGramMaxSplits);
    if (need > c->gram_floats) {
        KVMAP_HIP(hipDeviceSynchronize());
        (void)hipFree(c->gram);
        c->gram = nullptr;
        c->gram_floats = 0;
        KVMAP_HIP(hipMalloc((void**)&c->gram, need * sizeof(float)));
        c->gram_floats = need;
    }
    const size_t need_split = split_rows > 0 ? gram_split_elems(p, q, split_rows) : 0;
    if (need_split > c->gram_split_elems) {
        KVMAP_HIP(hipDeviceSynchronize());
        (void)hipFree(c->gram_split);
        c->gram_split = nullptr;
        c->gram_split_elems = 0;
        KVMAP_HIP(hipMalloc((void**)&c->gram_split, need_split * sizeof(uint16_t)));
        c->gram_split_elems = need_split;
    }
    return KVMAP_OK;
}

static GramScratch gram_scratch_at(float* base, uint16_t* split, int p, int q, int splits) {
    GramScratch sc;
    sc.part = base;
    base += (size_t)kGramMaxSplits * (p + q);
    sc.part2 = base;
    base += (size_t)kGramMaxSplits * (p + q);
    sc.cx = base; base += p;
    sc.cy = base; base += q;
    sc.mx = base; base += p;
    sc.my = base; base += q;
    sc.dx = base; base += p;
    sc.dy = base;
    sc.split = split;
    sc.splits = splits;
    sc.max_splits = kGramMaxSplits;
    return sc;
}

static GramScratch gram_scratch(kvmap_ctx* c, int p, int q, int splits) {
    return gram_scratch_at(c->gram, c->gram_split, p, q, splits);
}

// Host checks of a statistics call (no context involved); KVMAP_OK with *empty set for n_b = 0.
static int check_gram_args(const void* X, const void* Y, int64_t n_b, int32_t dtype, const kvmap_gram_state* st,
                           const char* who, bool* empty) {
    *empty = false;
    int r = validate_state(st, who);
    if (r) return r;
    if (dtype != KVMAP_DTYPE_BF16 && dtype != KVMAP_DTYPE_F32)
        return fail(KVMAP_ERR_UNSUPPORTED, "%s: dtype %d unknown", who, (int)dtype);
    if (n_b < 0 || n_b > (int64_t(1) << 31)) return fail(KVMAP_ERR_SHAPE, "%s: n_b out of range", who);
    if (n_b == 0) {
        *empty = true;
        return KVMAP_OK;
    }
    if (!X || !Y) return fail(KVMAP_ERR_INVALID_ARGUMENT, "%s: NULL batch", who);
    if ((((uintptr_t)X) | ((uintptr_t)Y)) & 15)
        return fail(KVMAP_ERR_INVALID_ARGUMENT, "%s: batch pointers must be 16-byte aligned", who);
    // the batch is read while the state is written: no overlap
    const size_t es = dtype == KVMAP_DTYPE_BF16 ? 2 : 4;
    const size_t xb = (size_t)n_b * st->p * es, yb = (size_t)n_b * st->q * es;
    const size_t p = (size_t)st->p, q = (size_t)st->q;
    const void* outs[5] = {st->mean_x, st->mean_y, st->M_xx, st->M_xy, st->ss_y};
    const size_t osz[5] = {p * 4, q * 4, p * (st->xx_block ? (size_t)st->xx_block : p) * 4, p * q * 4, q * 4};
    for (int i = 0; i < 5; ++i)
        if (outs[i] && (ranges_overlap(X, xb, outs[i], osz[i]) || ranges_overlap(Y, yb, outs[i], osz[i])))
            return fail(KVMAP_ERR_INVALID_ARGUMENT, "%s: the batch overlaps the state", who);
    return KVMAP_OK;
}

extern "C" int kvmap_validate_gram(const kvmap_gram_state* st, const void* X, const void* Y, int64_t n_b,
                                   int32_t dtype) {
    bool empty = false;
    const int r = check_gram_args(X, Y, n_b, dtype, st, "kvmap_gram", &empty);
    return r ? r : ok();
}

// Checks shared by kvmap_gram and kvmap_gram_noalloc; KVMAP_OK with *empty set for n_b = 0.
static int check_gram_call(kvmap_ctx* c, const void* X, const void* Y, int64_t n_b, int32_t dtype,
                           const kvmap_gram_state* st, const char* who, bool* empty) {
    *empty = false;
    if (!c) return fail(KVMAP_ERR_INVALID_ARGUMENT, "%s: ctx is NULL", who);
    return check_gram_args(X, Y, n_b, dtype, st, who, empty);
}

// The batch merged in sub-batches of at most `sub` rows (Chan merges compose exactly), each
// through the scratch at fbase (floats) and split (bf16 operands).
static int run_gram(const void* X, const void* Y, int64_t n_b, Elem e, kvmap_gram_state* st, int64_t sub,
                    float* fbase, uint16_t* split, hipStream_t s) {
    const size_t esz = e == Elem::BF16 ? 2 : 4;
    for (int64_t r0 = 0; r0 < n_b; r0 += sub) {
        const int64_t nr = std::min<int64_t>(sub, n_b - r0);
        const int splits = (int)std::min<int64_t>(kGramMaxSplits, std::max<int64_t>(1, nr / 64));
        const GramScratch sc = gram_scratch_at(fbase, split, st->p, st->q, splits);
        const char* xb = (const char*)X + (size_t)r0 * st->p * esz;
        const char* yb = (const char*)Y + (size_t)r0 * st->q * esz;
        KVMAP_HIP(launch_gram_batch(e, xb, yb, nr, st->p, st->q, st->n, st->mean_x, st->mean_y, st->M_xx, st->M_xy,
                                    st->ss_y, st->xx_block, sc, s));
        st->n += nr;
    }
    return KVMAP_OK;
}

extern "C" int kvmap_gram_reset(kvmap_ctx* c, kvmap_gram_state* st, void* stream) {
    if (!c) return fail(KVMAP_ERR_INVALID_ARGUMENT, "kvmap_gram_reset: ctx is NULL");
    int r = validate_state(st, "kvmap_gram_reset");
    if (r) return r;
    DeviceGuard g(c->device);
    hipStream_t s = (hipStream_t)stream;
    KVMAP_HIP(launch_fill_zero(st->mean_x, st->p, s));
    KVMAP_HIP(launch_fill_zero(st->mean_y, st->q, s));
    KVMAP_HIP(launch_fill_zero(st->M_xx, (int64_t)st->p * (st->xx_block ? st->xx_block : st->p), s));
    KVMAP_HIP(launch_fill_zero(st->M_xy, (int64_t)st->p * st->q, s));
    if (st->ss_y) KVMAP_HIP(launch_fill_zero(st->ss_y, st->q, s));
    st->n = 0;
    return ok();
}

extern "C" int kvmap_gram(kvmap_ctx* c, const void* X, const void* Y, int64_t n_b, int32_t dtype,
                          kvmap_gram_state* st, void* stream) {
    bool empty = false;
    int r = check_gram_call(c, X, Y, n_b, dtype, st, "kvmap_gram", &empty);
    if (r || empty) return r ? r : ok();
    DeviceGuard g(c->device);
    const Elem e = dtype == KVMAP_DTYPE_BF16 ? Elem::BF16 : Elem::F32;
    const int64_t sub = e == Elem::BF16 ? std::min<int64_t>(n_b, kGramSubBatch) : n_b;
    r = ensure_gram_scratch(c, st->p, st->q, e == Elem::BF16 ? sub : 0);
    if (r) return r;
    r = run_gram(X, Y, n_b, e, st, sub, c->gram, c->gram_split, (hipStream_t)stream);
    return r ? r : ok();
}

// Rows of one sub-batch that fit the static scratch next to its fixed part (0: not even 32).
static int64_t static_scratch_rows(int p, int q, Elem e, int64_t n_b) {
    const size_t fixed = (gram_scratch_floats(p, q, kGramMaxSplits) * sizeof(float) + 255) & ~(size_t)255;
    if (fixed > KVMAP_STATIC_SCRATCH_BYTES) return 0;
    if (e == Elem::F32) return n_b;  // the fp32 path keeps no per-row scratch
    const size_t per32 = gram_split_elems(p, q, 32) * sizeof(uint16_t);  // one 32-row block
    const int64_t blocks = (int64_t)((KVMAP_STATIC_SCRATCH_BYTES - fixed) / per32);
    return std::min<int64_t>(std::min<int64_t>(blocks * 32, kGramSubBatch), n_b);
}

extern "C" int kvmap_gram_noalloc(kvmap_ctx* c, const void* X, const void* Y, int64_t n_b, int32_t dtype,
                                  kvmap_gram_state* st, void* stream) {
    bool empty = false;
    int r = check_gram_call(c, X, Y, n_b, dtype, st, "kvmap_gram_noalloc", &empty);
    if (r || empty) return r ? r : ok();
    const Elem e = dtype == KVMAP_DTYPE_BF16 ? Elem::BF16 : Elem::F32;
    const int64_t sub = static_scratch_rows(st->p, st->q, e, n_b);
    if (sub < 1)
        return fail(KVMAP_ERR_UNSUPPORTED,
                    "kvmap_gram_noalloc: p + q = %d needs more than the %zu-byte static scratch (its fixed part is "
                    "%zu bytes, plus %zu per 32 rows for bf16); use kvmap_gram",
                    st->p + st->q, (size_t)KVMAP_STATIC_SCRATCH_BYTES,
                    gram_scratch_floats(st->p, st->q, kGramMaxSplits) * sizeof(float),
                    gram_split_elems(st->p, st->q, 32) * sizeof(uint16_t));
    if (!c->static_scratch) return fail(KVMAP_ERR_DEVICE, "kvmap_gram_noalloc: static scratch not resolved");
    DeviceGuard g(c->device);
    // [0, fixed): the float scratch (split partial sums, shift, means, deltas); then the bf16
    // operands of one sub-batch.  Every kernel writes what it reads first (padding rows of the
    // last 32-row block included), so nothing has to be cleared between calls.
    float* fbase = (float*)c->static_scratch;
    const size_t fixed = (gram_scratch_floats(st->p, st->q, kGramMaxSplits) * sizeof(float) + 255) & ~(size_t)255;
    uint16_t* split = (uint16_t*)((char*)c->static_scratch + fixed);
    r = run_gram(X, Y, n_b, e, st, sub, fbase, split, (hipStream_t)stream);
    return r ? r : ok();
}

extern "C" int kvmap_gram_merge(kvmap_ctx* c, kvmap_gram_state* dst, const kvmap_gram_state* src,
                                void* stream) {
    if (!c) return fail(KVMAP_ERR_INVALID_ARGUMENT, "kvmap_gram_merge: ctx is NULL");
    int r = validate_state(dst, "kvmap_gram_merge dst");
    if (r) return r;
    r = validate_state(src, "kvmap_gram_merge src");
    if (r) return r;
    if (dst->p != src->p || dst->q != src->q)
        return fail(KVMAP_ERR_SHAPE, "kvmap_gram_merge: p/q differ");
    if (!dst->ss_y != !src->ss_y)
        return fail(KVMAP_ERR_INVALID_ARGUMENT, "kvmap_gram_merge: ss_y kept by one state only");
    if (dst->xx_block != src->xx_block)
        return fail(KVMAP_ERR_SHAPE, "kvmap_gram_merge: xx_block differs");
    {
        // dst is written while src is read: no array of one may overlap an array of the other
        const size_t p = (size_t)dst->p, q = (size_t)dst->q, bx = dst->xx_block ? (size_t)dst->xx_block : p;
        const size_t sz[5] = {p * 4, q * 4, p * bx * 4, p * q * 4, q * 4};
        const void* da[5] = {dst->mean_x, dst->mean_y, dst->M_xx, dst->M_xy, dst->ss_y};
        const void* sa[5] = {src->mean_x, src->mean_y, src->M_xx, src->M_xy, src->ss_y};
        for (int i = 0; i < 5; ++i)
            for (int j = 0; j < 5; ++j)
                if (da[i] && sa[j] && ranges_overlap(da[i], sz[i], sa[j], sz[j]))
                    return fail(KVMAP_ERR_INVALID_ARGUMENT, "kvmap_gram_merge: dst and src overlap");
    }
    if (src->n == 0) return ok();
    DeviceGuard g(c->device);
    r = ensure_gram_scratch(c, dst->p, dst->q, 0);
    if (r) return r;
    const GramScratch sc = gram_scratch(c, dst->p, dst->q, 1);
    KVMAP_HIP(launch_gram_merge(dst->p, dst->q, dst->n, src->n, dst->mean_x, dst->mean_y, dst->M_xx,
                                dst->M_xy, dst->ss_y, src->mean_x, src->mean_y, src->M_xx, src->M_xy,
                                src->ss_y, dst->xx_block, sc,
                                (hipStream_t)stream));
    dst->n += src->n;
    return ok();
}

// ---------------------------------------------------------------------------------------
// ridge solve
// ---------------------------------------------------------------------------------------

extern "C" int kvmap_ridge_solve_host(int32_t p, int32_t q, const float* mean_x, const float* mean_y,
                                      const float* M_xx, const float* M_xy, double lambda, float* W_out,
                                      float* b_out, int n_threads) {
    if (p < 1 || q < 1) return fail(KVMAP_ERR_SHAPE, "kvmap_ridge_solve_host: p, q must be >= 1");
    if (!mean_x || !mean_y || !M_xx || !M_xy || !W_out || !b_out)
        return fail(KVMAP_ERR_INVALID_ARGUMENT, "kvmap_ridge_solve_host: NULL pointer");
    if (!(lambda >= 0.0) || !std::isfinite(lambda))
        return fail(KVMAP_ERR_INVALID_ARGUMENT, "kvmap_ridge_solve_host: lambda must be finite and >= 0");
    int r;
    try {  // the fp64 system takes p^2 * 8 bytes of host memory (32 GiB at p 65,536)
        r = ridge_solve_f64(p, q, mean_x, mean_y, M_xx, M_xy, lambda, W_out, b_out, n_threads);
    } catch (const std::bad_alloc&) {
        return fail(KVMAP_ERR_OUT_OF_MEMORY, "kvmap_ridge_solve_host: no host memory for the fp64 system");
    }
    if (r) return fail(KVMAP_ERR_NOT_SPD, "kvmap_ridge_solve_host: M_xx + lambda I is not positive definite");
    return ok();
}

static int ensure_ridge_scratch(kvmap_ctx* c, size_t need) {
    if (!c->ridge_ov.side) {  // the lookahead's side stream (default priority) and its events
        KVMAP_HIP(hipStreamCreateWithFlags(&c->ridge_ov.side, hipStreamNonBlocking));
        KVMAP_HIP(hipEventCreateWithFlags(&c->ridge_ov.main_ready, hipEventDisableTiming));
        KVMAP_HIP(hipEventCreateWithFlags(&c->ridge_ov.side_done, hipEventDisableTiming));
        KVMAP_HIP(hipEventCreateWithFlags(&c->ridge_ov.side_done2, hipEventDisableTiming));
        KVMAP_HIP(hipStreamCreateWithFlags(&c->ridge_ov.fwd, hipStreamNonBlocking));
        KVMAP_HIP(hipEventCreateWithFlags(&c->ridge_ov.fwd_ready, hipEventDisableTiming));
        KVMAP_HIP(hipEventCreateWithFlags(&c->ridge_ov.fwd_done, hipEventDisableTiming));
    }
    if (need > c->ridge_bytes) {
        KVMAP_HIP(hipDeviceSynchronize());
        (void)hipFree(c->ridge);
        c->ridge = nullptr;
        c->ridge_bytes = 0;
        KVMAP_HIP(hipMalloc(&c->ridge, need));
        c->ridge_bytes = need;
    }
    return KVMAP_OK;
}

// The device solves of n states of one (p, q), in batches of up to kRidgeMaxBatch systems that
// share one scratch of at most about kRidgeScratchBudget bytes (at least one system).  Each
// batch is checked for non-positive pivots before the next starts.  r2: R^2 per group of y
// columns into r2o[i]; else W[i], b[i] in bf16 or fp32.
constexpr size_t kRidgeScratchBudget = size_t(16) << 30;

static int run_ridge(kvmap_ctx* c, const kvmap_gram_state* const* st, int n, double lambda, bool r2, int group,
                     bool bf16, void* const* W, void* const* b, double* const* r2o, hipStream_t s, const char* who) {
    const int p = st[0]->p, q = st[0]->q;
    const size_t per = ridge_dev_scratch_bytes(p, q, 1) - 256;
    const int chunk = (int)std::min<size_t>(std::min<size_t>(kRidgeMaxBatch, (size_t)n),
                                            std::max<size_t>(1, kRidgeScratchBudget / per));
    int r = ensure_ridge_scratch(c, ridge_dev_scratch_bytes(p, q, chunk));
    if (r) return r;
    int flags[kRidgeMaxBatch];
    for (int i0 = 0; i0 < n; i0 += chunk) {
        const int m = std::min(chunk, n - i0);
        RidgeSys sys[kRidgeMaxBatch];
        for (int j = 0; j < m; ++j) {
            const kvmap_gram_state* t = st[i0 + j];
            sys[j] = RidgeSys{t->M_xx, t->M_xy, t->mean_x, t->mean_y, t->ss_y,
                              r2 ? nullptr : W[i0 + j], r2 ? nullptr : b[i0 + j], r2 ? r2o[i0 + j] : nullptr};
        }
        int* bad = ridge_dev_flags(c->ridge, p, q, m);
        KVMAP_HIP(launch_fill_zero((float*)bad, m, s));
        if (r2) KVMAP_HIP(launch_ridge_r2(m, p, q, sys, lambda, group, c->ridge, s, c->ridge_ov));
        else KVMAP_HIP(launch_ridge_dev(m, p, q, sys, lambda, bf16, c->ridge, s, c->ridge_ov));
        KVMAP_HIP(hipMemcpyAsync(flags, bad, m * sizeof(int), hipMemcpyDeviceToHost, s));
        KVMAP_HIP(hipStreamSynchronize(s));
        for (int j = 0; j < m; ++j)
            if (flags[j])
                return fail(KVMAP_ERR_NOT_SPD, "%s: system %d: M_xx + lambda I is not positive definite", who, i0 + j);
    }
    return KVMAP_OK;
}

// Arguments of one device solve (state, outputs): nothing written when refused.
static int check_solve_args(const kvmap_gram_state* st, const void* W_out, const void* b_out, int32_t dtype,
                            const char* who) {
    int r = validate_state(st, who);
    if (r) return r;
    if (st->xx_block) return fail(KVMAP_ERR_UNSUPPORTED, "%s: a block-diagonal state (solve its blocks' views)", who);
    if (!W_out || !b_out) return fail(KVMAP_ERR_INVALID_ARGUMENT, "%s: NULL output", who);
    const size_t es = dtype == KVMAP_DTYPE_BF16 ? 2 : 4;
    const size_t wb = (size_t)st->p * st->q * es, bb = (size_t)st->q * es;
    if ((((uintptr_t)W_out) | ((uintptr_t)b_out)) & 3)
        return fail(KVMAP_ERR_INVALID_ARGUMENT, "%s: outputs must be 4-byte aligned", who);
    if (ranges_overlap(W_out, wb, b_out, bb)) return fail(KVMAP_ERR_INVALID_ARGUMENT, "%s: W_out and b_out overlap", who);
    const void* ins[4] = {st->mean_x, st->mean_y, st->M_xx, st->M_xy};
    const size_t insz[4] = {(size_t)st->p * 4, (size_t)st->q * 4, (size_t)st->p * st->p * 4, (size_t)st->p * st->q * 4};
    for (int i = 0; i < 4; ++i)
        if (ranges_overlap(ins[i], insz[i], W_out, wb) || ranges_overlap(ins[i], insz[i], b_out, bb))
            return fail(KVMAP_ERR_INVALID_ARGUMENT, "%s: an output overlaps the state", who);
    return KVMAP_OK;
}

static int check_r2_args(const kvmap_gram_state* st, int32_t group, const double* r2_out, const char* who) {
    int r = validate_state(st, who);
    if (r) return r;
    if (st->xx_block) return fail(KVMAP_ERR_UNSUPPORTED, "%s: a block-diagonal state (solve its blocks' views)", who);
    if (!st->ss_y) return fail(KVMAP_ERR_INVALID_ARGUMENT, "%s: the state keeps no ss_y", who);
    if (!r2_out) return fail(KVMAP_ERR_INVALID_ARGUMENT, "%s: NULL output", who);
    if (group < 1 || st->q % group)
        return fail(KVMAP_ERR_SHAPE, "%s: group %d must divide q = %d", who, (int)group, (int)st->q);
    if (((uintptr_t)r2_out) & 7) return fail(KVMAP_ERR_INVALID_ARGUMENT, "%s: r2_out must be 8-byte aligned", who);
    const size_t ob = (size_t)(st->q / group) * 8;
    const void* ins[5] = {st->mean_x, st->mean_y, st->M_xx, st->M_xy, st->ss_y};
    const size_t insz[5] = {(size_t)st->p * 4, (size_t)st->q * 4, (size_t)st->p * st->p * 4,
                            (size_t)st->p * st->q * 4, (size_t)st->q * 4};
    for (int i = 0; i < 5; ++i)
        if (ranges_overlap(ins[i], insz[i], r2_out, ob))
            return fail(KVMAP_ERR_INVALID_ARGUMENT, "%s: r2_out overlaps the state", who);
    return KVMAP_OK;
}

static int check_common(kvmap_ctx* c, double lambda, const char* who) {
    if (!c) return fail(KVMAP_ERR_INVALID_ARGUMENT, "%s: ctx is NULL", who);
    if (!(lambda >= 0.0) || !std::isfinite(lambda))
        return fail(KVMAP_ERR_INVALID_ARGUMENT, "%s: lambda must be finite and >= 0", who);
    return KVMAP_OK;
}

extern "C" int kvmap_ridge_solve_device(kvmap_ctx* c, const kvmap_gram_state* st, double lambda, void* W_out,
                                        void* b_out, int32_t dtype, void* stream) {
    const char* who = "kvmap_ridge_solve_device";
    int r = check_common(c, lambda, who);
    if (r) return r;
    if (dtype != KVMAP_DTYPE_BF16 && dtype != KVMAP_DTYPE_F32)
        return fail(KVMAP_ERR_UNSUPPORTED, "%s: dtype %d unknown", who, (int)dtype);
    r = check_solve_args(st, W_out, b_out, dtype, who);
    if (r) return r;
    DeviceGuard g(c->device);
    r = run_ridge(c, &st, 1, lambda, false, 0, dtype == KVMAP_DTYPE_BF16, &W_out, &b_out, nullptr,
                  (hipStream_t)stream, who);
    return r ? r : ok();
}

extern "C" int kvmap_ridge_solve_device_batch(kvmap_ctx* c, const kvmap_gram_state* const* states, int32_t n,
                                              double lambda, void* const* W_out, void* const* b_out, int32_t dtype,
                                              void* stream) {
    const char* who = "kvmap_ridge_solve_device_batch";
    int r = check_common(c, lambda, who);
    if (r) return r;
    if (dtype != KVMAP_DTYPE_BF16 && dtype != KVMAP_DTYPE_F32)
        return fail(KVMAP_ERR_UNSUPPORTED, "%s: dtype %d unknown", who, (int)dtype);
    if (n < 1 || !states || !W_out || !b_out) return fail(KVMAP_ERR_INVALID_ARGUMENT, "%s: empty batch or NULL array", who);
    const size_t es = dtype == KVMAP_DTYPE_BF16 ? 2 : 4;
    for (int i = 0; i < n; ++i) {
        r = check_solve_args(states[i], W_out[i], b_out[i], dtype, who);
        if (r) return r;
        if (states[i]->p != states[0]->p || states[i]->q != states[0]->q)
            return fail(KVMAP_ERR_SHAPE, "%s: state %d has another (p, q) than state 0", who, i);
        const size_t wb = (size_t)states[i]->p * states[i]->q * es, bb = (size_t)states[i]->q * es;
        for (int j = 0; j < i; ++j) {
            if (ranges_overlap(W_out[i], wb, W_out[j], wb) || ranges_overlap(W_out[i], wb, b_out[j], bb) ||
                ranges_overlap(b_out[i], bb, W_out[j], wb) || ranges_overlap(b_out[i], bb, b_out[j], bb))
                return fail(KVMAP_ERR_INVALID_ARGUMENT, "%s: outputs of systems %d and %d overlap", who, j, i);
        }
    }
    DeviceGuard g(c->device);
    r = run_ridge(c, states, n, lambda, false, 0, dtype == KVMAP_DTYPE_BF16, W_out, b_out, nullptr,
                  (hipStream_t)stream, who);
    return r ? r : ok();
}

extern "C" int kvmap_ridge_r2(kvmap_ctx* c, const kvmap_gram_state* st, double lambda, int32_t group,
                              double* r2_out, void* stream) {
    const char* who = "kvmap_ridge_r2";
    int r = check_common(c, lambda, who);
    if (r) return r;
    r = check_r2_args(st, group, r2_out, who);
    if (r) return r;
    DeviceGuard g(c->device);
    r = run_ridge(c, &st, 1, lambda, true, group, false, nullptr, nullptr, &r2_out, (hipStream_t)stream, who);
    return r ? r : ok();
}

extern "C" int kvmap_ridge_r2_batch(kvmap_ctx* c, const kvmap_gram_state* const* states, int32_t n, double lambda,
                                    int32_t group, double* const* r2_out, void* stream) {
    const char* who = "kvmap_ridge_r2_batch";
    int r = check_common(c, lambda, who);
    if (r) return r;
    if (n < 1 || !states || !r2_out) return fail(KVMAP_ERR_INVALID_ARGUMENT, "%s: empty batch or NULL array", who);
    for (int i = 0; i < n; ++i) {
        r = check_r2_args(states[i], group, r2_out[i], who);
        if (r) return r;
        if (states[i]->p != states[0]->p || states[i]->q != states[0]->q)
            return fail(KVMAP_ERR_SHAPE, "%s: state %d has another (p, q) than state 0", who, i);
        const size_t ob = (size_t)(states[i]->q / group) * 8;
        for (int j = 0; j < i; ++j)
            if (ranges_overlap(r2_out[i], ob, r2_out[j], ob))
                return fail(KVMAP_ERR_INVALID_ARGUMENT, "%s: outputs of systems %d and %d overlap", who, j, i);
    }
    DeviceGuard g(c->device);
    r = run_ridge(c, states, n, lambda, true, group, false, nullptr, nullptr, r2_out, (hipStream_t)stream, who);
    return r ? r : ok();
}

extern "C" int kvmap_ridge_solve(kvmap_ctx* c, const kvmap_gram_state* st, double lambda, float* W_out,
                                 float* b_out, void* stream) {
    if (!c) return fail(KVMAP_ERR_INVALID_ARGUMENT, "kvmap_ridge_solve: ctx is NULL");
    int r = validate_state(st, "kvmap_ridge_solve");
    if (r) return r;
    if (st->xx_block) return fail(KVMAP_ERR_UNSUPPORTED, "kvmap_ridge_solve: a block-diagonal state");
    if (!W_out || !b_out) return fail(KVMAP_ERR_INVALID_ARGUMENT, "kvmap_ridge_solve: NULL output");
    DeviceGuard g(c->device);
    const size_t p = st->p, q = st->q;
    std::vector<float> mx, my, Mxx, Mxy;
    try {
        mx.resize(p);
        my.resize(q);
        Mxx.resize(p * p);
        Mxy.resize(p * q);
    } catch (const std::bad_alloc&) {
        return fail(KVMAP_ERR_OUT_OF_MEMORY, "kvmap_ridge_solve: no host memory for the statistics");
    }
    hipStream_t s = (hipStream_t)stream;
    KVMAP_HIP(hipMemcpyAsync(mx.data(), st->mean_x, p * 4, hipMemcpyDeviceToHost, s));
    KVMAP_HIP(hipMemcpyAsync(my.data(), st->mean_y, q * 4, hipMemcpyDeviceToHost, s));
    KVMAP_HIP(hipMemcpyAsync(Mxx.data(), st->M_xx, p * p * 4, hipMemcpyDeviceToHost, s));
    KVMAP_HIP(hipMemcpyAsync(Mxy.data(), st->M_xy, p * q * 4, hipMemcpyDeviceToHost, s));
    KVMAP_HIP(hipStreamSynchronize(s));
    return kvmap_ridge_solve_host(st->p, st->q, mx.data(), my.data(), Mxx.data(), Mxy.data(), lambda, W_out,
                                  b_out, 0);
}
