// host.cpp -- the C ABI of libmmq: context, plane cache, registration and
// dispatch.  Declarations and the contract of every entry point: include/mmq.h.
//
// Plane cache ("55 · r52 ...", sections 3.1-3.2; "72 · D3-7 ...", Excerpts A2,
// C and D).  Producers record the plane they wrote under the f32 buffer they
// produced (or, with write_y = 0, the buffer they were promised but never
// wrote); consumers look the plane up by (pointer, n, d) and on a miss
// quantise the buffer themselves and record it.  A skip-write producer marks
// its output range dead: any later request that would read bytes of a dead
// range -- a quantise, or a producer taking it as an input -- refuses loudly
// (status MMQ_E_DEAD_WRITE plus one stderr line) instead of reading memory
// that was never written.  Every write the library makes to caller memory (a
// producer's y, a consumer's out, an export) drops the cached planes whose
// key bytes it overwrites and revives the dead bytes it defines.
// mmq_cache_clear is the execution-window boundary: it drops every entry and
// every dead range.
//
// The table has kSlots entries, each owning one grow-only device plane slot;
// when all are in use the least recently used entry is evicted and its slot
// reused.  All launches go to the caller's stream in call order, so a slot is
// only rewritten after every earlier kernel that read it (same stream).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "mmq.h"
#include "mmq_internal.h"

using namespace mmq;

// The one-token plane of the allocation-free decode call (mmvq_q6k_noalloc):
// a file-scope device array, one copy per GPU, held until the process ends.
// Layout as a plane of one row: codes [kStaticMaxCols], then the (D, S) pairs
// at byte kStaticMaxCols.  Host code never uses the array's name as an
// address: the per-device address comes from hipGetSymbolAddress.
constexpr int64_t kStaticMaxCols = MMQ_NOALLOC_MAX_COLS;
constexpr int64_t kStaticPlaneBytes = kStaticMaxCols + kStaticMaxCols / kBlock * 8;
static __device__ __align__(256) unsigned char scratch[kStaticPlaneBytes];

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

constexpr int kSlots = 8;

struct Entry {
    bool used = false;
    const void* key = nullptr;
    int64_t n = 0, d = 0;
    bool dead = false;
    uint64_t last = 0;
};

struct Slot {
    void* mem = nullptr;
    int64_t cap = 0;
};

struct DeadRange {
    uintptr_t lo, hi;  // [lo, hi)
    uintptr_t key;     // the skip-write producer output it was recorded for
};

int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

int64_t plane_bytes_for(int64_t n, int64_t d, int64_t* off_ds) {
    const int64_t rows = round_up(n, kPlaneRows);
    const int64_t nb = d / kBlock;
    const int64_t o = round_up(rows * d, 256);
    if (off_ds) *off_ds = o;
    return o + round_up(rows * nb * 8, 256);
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

std::mutex g_scratch_mu;
std::map<int, void*> g_scratch_ptr;   // device -> address of `scratch` there

// Address of `scratch` on `device`, which must be current; resolved once per
// device.
int scratch_address(int device, void** out) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    auto it = g_scratch_ptr.find(device);
    if (it == g_scratch_ptr.end()) {
        void* ptr = nullptr;
        hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || ptr == nullptr) {
            (void)hipGetLastError();
            return fail(MMQ_E_HIP, "hipGetSymbolAddress(scratch) on device %d: HIP error %d (%s)",
                        device, (int)e, hipGetErrorString(e));
        }
        it = g_scratch_ptr.emplace(device, ptr).first;
    }
    *out = it->second;
    return MMQ_OK;
}

}  // namespace

struct mmq_ctx {
    int device = -1;
    unsigned flags = 0;
    bool dry = false;
    int64_t cap = -1;
    Entry entries[kSlots];
    Slot slots[kSlots];
    std::vector<DeadRange> dead;
    uint64_t tick = 0;
    int64_t plane_bytes = 0;
    int64_t weight_bytes = 0;
    mmq_stats_t st{};
    // Once any call was captured into a graph, slot memory the graph may
    // reference is never freed before mmq_destroy: a grown slot's old memory
    // is retired here instead.
    bool captured = false;
    std::vector<void*> retired;
    // Registration-time consumer-set predicate: true while every consumer of
    // producer outputs reads planes.  A consumer that reads the f32 output
    // directly (declared with mmq_register_foreign_consumer) clears it, and
    // skip-write producers then degrade to writing y.
    bool plane_only = true;
    int n_cu = 256;              // compute units (K-split heuristic)
    void* part = nullptr;        // K-split partial outputs, grow-only
    int64_t part_cap = 0;
    void* static_plane = nullptr;  // this device's copy of `scratch`
};

struct mmq_weight {
    mmq_ctx* ctx = nullptr;
    bool dry = false;
    WeightDev w;
};

namespace {

int hip_fail(hipError_t e, const char* what) {
    return fail(MMQ_E_HIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

// True while `s` is being captured into a HIP graph (launches are recorded,
// not run; synchronising or allocating is not allowed).
bool capturing(const mmq_ctx* c, hipStream_t s) {
    if (c->dry) return false;
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &st) != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    return st == hipStreamCaptureStatusActive;
}

int after_launch(mmq_ctx* c, hipError_t e, hipStream_t s, const char* what) {
    if (e != hipSuccess) return hip_fail(e, what);
    if ((c->flags & MMQ_CTX_SYNC_CHECK) && !capturing(c, s)) {
        e = hipStreamSynchronize(s);
        if (e == hipSuccess) e = hipGetLastError();
        if (e != hipSuccess) return hip_fail(e, what);
    }
    return MMQ_OK;
}

int use_device(mmq_ctx* c) {
    if (c->dry) return MMQ_OK;
    hipError_t e = hipSetDevice(c->device);
    if (e != hipSuccess) return hip_fail(e, "hipSetDevice");
    return MMQ_OK;
}

bool overlaps_dead(const mmq_ctx* c, const void* p, int64_t bytes) {
    const uintptr_t lo = (uintptr_t)p, hi = lo + (uintptr_t)bytes;
    for (const DeadRange& r : c->dead)
        if (lo < r.hi && r.lo < hi) return true;
    return false;
}

int refuse_dead(mmq_ctx* c, const char* who, const void* p) {
    c->st.cache_refusals++;
    fprintf(stderr,
            "libmmq: %s refused: buffer %p was promised unread by a skip-write producer "
            "(write_y=0) and never written; quantising it would read garbage\n",
            who, p);
    return fail(MMQ_E_DEAD_WRITE, "%s: buffer %p overlaps a dead (never written) producer output",
                who, p);
}

// Remove [p, p + bytes) from every dead range (ranges are split if needed).
void revive(mmq_ctx* c, const void* p, int64_t bytes) {
    const uintptr_t lo = (uintptr_t)p, hi = lo + (uintptr_t)bytes;
    std::vector<DeadRange> keep;
    for (const DeadRange& r : c->dead) {
        if (hi <= r.lo || r.hi <= lo) {
            keep.push_back(r);
            continue;
        }
        if (r.lo < lo) keep.push_back({r.lo, lo, r.key});
        if (hi < r.hi) keep.push_back({hi, r.hi, r.key});
    }
    c->dead.swap(keep);
}

// [p, p + bytes) becomes a dead range recorded for key p (overlapping older
// ranges give up those bytes first, so the list stays disjoint).
void mark_dead(mmq_ctx* c, const void* p, int64_t bytes) {
    revive(c, p, bytes);
    c->dead.push_back({(uintptr_t)p, (uintptr_t)p + (uintptr_t)bytes, (uintptr_t)p});
}

int find_entry(const mmq_ctx* c, const void* key, int64_t n, int64_t d) {
    for (int i = 0; i < kSlots; ++i) {
        const Entry& e = c->entries[i];
        if (e.used && e.key == key && e.n == n && e.d == d) return i;
    }
    return -1;
}

// Drop entries whose key range overlaps [p, p + bytes): their planes describe
// contents that a producer is about to replace.
void drop_overlapping(mmq_ctx* c, const void* p, int64_t bytes) {
    const uintptr_t lo = (uintptr_t)p, hi = lo + (uintptr_t)bytes;
    for (Entry& e : c->entries) {
        if (!e.used) continue;
        const uintptr_t elo = (uintptr_t)e.key, ehi = elo + (uintptr_t)(e.n * e.d * 4);
        if (lo < ehi && elo < hi) e.used = false;
    }
}

// The library is about to write [p, p + bytes) of caller memory: planes keyed
// by those bytes describe old contents, and dead bytes become written.
void written(mmq_ctx* c, const void* p, int64_t bytes) {
    drop_overlapping(c, p, bytes);
    revive(c, p, bytes);
}

// Pick an entry for (key, n, d), growing its slot if needed.  The entry is
// not marked used until the caller commits it.
int acquire_slot(mmq_ctx* c, const void* key, int64_t n, int64_t d, bool in_capture,
                 int* out_idx) {
    int idx = find_entry(c, key, n, d);
    if (idx < 0) {
        for (int i = 0; i < kSlots && idx < 0; ++i)
            if (!c->entries[i].used) idx = i;
        if (idx < 0) {
            idx = 0;
            for (int i = 1; i < kSlots; ++i)
                if (c->entries[i].last < c->entries[idx].last) idx = i;
        }
    }
    const int64_t need = plane_bytes_for(n, d, nullptr);
    Slot& s = c->slots[idx];
    if (s.cap < need) {
        if (in_capture)
            return fail(MMQ_E_ARG,
                        "plane slot must grow to %lld bytes during stream capture, where nothing "
                        "may be allocated; make the same calls once before capturing",
                        (long long)need);
        const int64_t total = c->plane_bytes - s.cap + need;
        if (c->cap >= 0 && total > c->cap)
            return fail(MMQ_E_OOM, "plane scratch cap %lld bytes exceeded (need %lld in total)",
                        (long long)c->cap, (long long)total);
        if (!c->dry) {
            if (s.mem && c->captured) {
                c->retired.push_back(s.mem);  // a captured graph may still use it
                s.mem = nullptr;
            } else if (s.mem) {
                hipError_t e = hipFree(s.mem);
                if (e != hipSuccess) return hip_fail(e, "hipFree(plane slot)");
                s.mem = nullptr;
            }
            void* m = nullptr;
            hipError_t e = hipMalloc(&m, (size_t)need);
            if (e != hipSuccess) {
                // the slot lost its memory: whatever entry used it is gone too
                c->entries[idx].used = false;
                c->plane_bytes -= s.cap;
                s.cap = 0;
                (void)hipGetLastError();
                return fail(MMQ_E_OOM, "hipMalloc of a %lld-byte plane slot failed", (long long)need);
            }
            s.mem = m;
        }
        c->plane_bytes += need - s.cap;
        s.cap = need;
    }
    *out_idx = idx;
    return MMQ_OK;
}

void commit_entry(mmq_ctx* c, int idx, const void* key, int64_t n, int64_t d, bool dead) {
    Entry& e = c->entries[idx];
    e.used = true;
    e.key = key;
    e.n = n;
    e.d = d;
    e.dead = dead;
    e.last = ++c->tick;
}

PlaneView view_of(const mmq_ctx* c, int idx) {
    const Entry& e = c->entries[idx];
    int64_t o;
    plane_bytes_for(e.n, e.d, &o);
    char* base = (char*)c->slots[idx].mem;
    PlaneView v;
    v.q = (int8_t*)base;
    v.ds = (uint2*)(base + o);
    v.rows = round_up(e.n, kPlaneRows);
    v.d = e.d;
    return v;
}

int check_nd(const char* who, int64_t n, int64_t d) {
    if (n < 1) return fail(MMQ_E_SHAPE, "%s: n=%lld must be >= 1", who, (long long)n);
    if (d < kSuper || d % kSuper != 0)
        return fail(MMQ_E_SHAPE, "%s: d=%lld must be a positive multiple of 256", who,
                    (long long)d);
    if (round_up(n, kPlaneRows) > (int64_t)1 << 30 || d > (int64_t)1 << 28 ||
        round_up(n, kPlaneRows) * d > ((int64_t)1 << 40))
        return fail(MMQ_E_SHAPE, "%s: n=%lld d=%lld too large", who, (long long)n, (long long)d);
    return MMQ_OK;
}

// Shared body of the three producers.
int produce(mmq_ctx* c, ProducerKind kind, const char* who, const float* a, const float* b,
            float* y, int64_t n, int64_t d, float eps, int write_y, void* stream) {
    if (!c) return fail(MMQ_E_ARG, "%s: null context", who);
    int rc = check_nd(who, n, d);
    if (rc) return rc;
    if (!a || !aligned16(a) || (kind != kProdF32 && (!b || !aligned16(b))) ||
        (kind != kProdF32 && (!y || !aligned16(y))))
        return fail(MMQ_E_ARG, "%s: null or non-16-byte-aligned pointer", who);
    if (kind != kProdF32 && write_y != 0 && write_y != 1 && write_y != MMQ_WRITE_AUTO)
        return fail(MMQ_E_ARG, "%s: write_y=%d (0, 1 or MMQ_WRITE_AUTO)", who, write_y);
    const int64_t bytes = n * d * 4;
    // every f32 input the kernel reads must have been written: x (or gate),
    // and the RMSNorm weight [d] or the SwiGLU up [n][d]
    if (overlaps_dead(c, a, bytes)) return refuse_dead(c, who, a);
    if (kind == kProdRms && overlaps_dead(c, b, d * 4)) return refuse_dead(c, who, b);
    if (kind == kProdSwiglu && overlaps_dead(c, b, bytes)) return refuse_dead(c, who, b);
    // The degradation ladder: skip-write (y never written) only while every
    // consumer reads planes; otherwise write y and the plane.
    const int auto_mode = write_y == MMQ_WRITE_AUTO;
    const bool want_skip = kind != kProdF32 && (write_y == 0 || write_y == MMQ_WRITE_AUTO);
    const bool skip = want_skip && c->plane_only;
    if (want_skip && !skip) c->st.degraded_writes++;
    write_y = kind == kProdF32 ? 0 : (skip ? 0 : 1);
    const void* key = kind == kProdF32 ? (const void*)a : (const void*)y;
    if ((rc = use_device(c))) return rc;
    int idx;
    // The producer replaces whatever was cached for bytes it (re)defines.
    drop_overlapping(c, kind != kProdF32 ? (const void*)y : (const void*)a, bytes);
    const bool in_capture = capturing(c, (hipStream_t)stream);
    if ((rc = acquire_slot(c, key, n, d, in_capture, &idx))) {
        // Last tier: with MMQ_WRITE_AUTO a producer that cannot get plane
        // memory writes y alone and records nothing; consumers then quantise
        // y themselves (and fail loudly if that cannot be done either).
        if (rc != MMQ_E_OOM || auto_mode == 0 || kind == kProdF32) return rc;
        c->st.unfused_fallbacks++;
        if (kind == kProdRms) c->st.launches_quant_rms++;
        else c->st.launches_quant_swiglu++;
        revive(c, y, bytes);
        fprintf(stderr, "libmmq: %s: no plane memory (%s); wrote y without a plane\n", who,
                mmq_last_error());
        if (c->dry) return MMQ_OK;
        hipStream_t s = (hipStream_t)stream;
        const PlaneView none{};
        return after_launch(c, launch_producer(kind, a, b, y, n, d, eps, true, none, s), s, who);
    }
    if (in_capture) c->captured = true;
    if (kind != kProdF32 && write_y) revive(c, y, bytes);  // a real write makes these bytes valid
    const bool dead = kind != kProdF32 && !write_y;
    commit_entry(c, idx, key, n, d, dead);
    if (dead) mark_dead(c, y, bytes);
    if (kind == kProdRms) c->st.launches_quant_rms++;
    else if (kind == kProdSwiglu) c->st.launches_quant_swiglu++;
    else c->st.launches_quant_f32++;
    if (c->dry) return MMQ_OK;
    hipStream_t s = (hipStream_t)stream;
    const PlaneView pl = view_of(c, idx);
    hipError_t e = launch_producer(kind, a, b, y, n, d, eps, write_y != 0, pl, s);
    return after_launch(c, e, s, who);
}

// Consumer side: the plane of (a, n, d), quantising it on a miss.
int plane_for(mmq_ctx* c, const char* who, const float* a, int64_t n, int64_t d, void* stream,
              PlaneView* out) {
    if (capturing(c, (hipStream_t)stream)) c->captured = true;
    int idx = find_entry(c, a, n, d);
    if (idx >= 0) {
        c->st.cache_hits++;
        c->entries[idx].last = ++c->tick;
        *out = c->dry ? PlaneView{} : view_of(c, idx);
        return MMQ_OK;
    }
    if (overlaps_dead(c, a, n * d * 4)) return refuse_dead(c, who, a);
    c->st.cache_misses++;
    int rc = produce(c, kProdF32, who, a, nullptr, nullptr, n, d, 0.0f, 0, stream);
    if (rc) return rc;
    idx = find_entry(c, a, n, d);
    *out = c->dry ? PlaneView{} : view_of(c, idx);
    return MMQ_OK;
}

int consume_check(mmq_ctx* c, const mmq_weight* w, const float* a, int64_t n, float* out,
                  int type, unsigned use, const char* who) {
    if (!c) return fail(MMQ_E_ARG, "%s: null context", who);
    if (!w || w->ctx != c) return fail(MMQ_E_ARG, "%s: weight is null or from another context", who);
    if (w->w.type != type)
        return fail(MMQ_E_TYPE, "%s: weight has type %d, this call needs %d", who, w->w.type, type);
    if (!(w->w.uses & use))
        return fail(MMQ_E_TYPE, "%s: weight was not registered for this consumer (uses=%u)", who,
                    w->w.uses);
    if (!a || !out || !aligned16(a) || !aligned16(out))
        return fail(MMQ_E_ARG, "%s: null or non-16-byte-aligned pointer", who);
    return check_nd(who, n, w->w.cols);
}

}  // namespace

extern "C" {

const char* mmq_last_error(void) { return g_err.c_str(); }

int64_t mmq_plane_rows(int64_t n) { return n < 1 ? 0 : round_up(n, kPlaneRows); }

int mmq_create(int device, unsigned flags, mmq_ctx** out) {
    if (!out) return fail(MMQ_E_ARG, "mmq_create: out is null");
    *out = nullptr;
    if (flags & ~(MMQ_CTX_SYNC_CHECK | MMQ_CTX_DRYRUN))
        return fail(MMQ_E_ARG, "mmq_create: unknown flags 0x%x", flags);
    mmq_ctx* c = new mmq_ctx();
    c->flags = flags;
    c->dry = (flags & MMQ_CTX_DRYRUN) != 0;
    if (!c->dry) {
        int count = 0;
        if (hipGetDeviceCount(&count) != hipSuccess || count <= 0 || device < 0 ||
            device >= count) {
            (void)hipGetLastError();
            delete c;
            return fail(MMQ_E_DEVICE, "mmq_create: no HIP device %d (found %d)", device, count);
        }
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, device) != hipSuccess) {
            delete c;
            return fail(MMQ_E_DEVICE, "mmq_create: cannot query device %d", device);
        }
        if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
            delete c;
            return fail(MMQ_E_DEVICE, "mmq_create: device %d is %s, this library is built for gfx950",
                        device, prop.gcnArchName);
        }
        if (hipSetDevice(device) != hipSuccess) {
            delete c;
            return fail(MMQ_E_DEVICE, "mmq_create: hipSetDevice(%d) failed", device);
        }
        if (int rc = scratch_address(device, &c->static_plane)) {
            delete c;
            return rc;
        }
        c->device = device;
        if (prop.multiProcessorCount > 0) c->n_cu = prop.multiProcessorCount;
    }
    *out = c;
    return MMQ_OK;
}

void mmq_destroy(mmq_ctx* c) {
    if (!c) return;
    if (!c->dry) {
        (void)hipSetDevice(c->device);
        (void)hipDeviceSynchronize();
        for (Slot& s : c->slots)
            if (s.mem) (void)hipFree(s.mem);
        for (void* p : c->retired) (void)hipFree(p);
        if (c->part) (void)hipFree(c->part);
    }
    delete c;
}

int mmq_set_scratch_cap(mmq_ctx* c, int64_t bytes) {
    if (!c) return fail(MMQ_E_ARG, "mmq_set_scratch_cap: null context");
    c->cap = bytes < 0 ? -1 : bytes;
    return MMQ_OK;
}

int mmq_register_weight(mmq_ctx* c, int type, int64_t rows, int64_t cols, const void* raw_host,
                        unsigned uses, mmq_weight** out) {
    const char* who = "mmq_register_weight";
    if (!c || !raw_host || !out) return fail(MMQ_E_ARG, "%s: null argument", who);
    *out = nullptr;
    if (type != MMQ_Q4_K && type != MMQ_Q5_K && type != MMQ_Q6_K)
        return fail(MMQ_E_TYPE, "%s: unsupported weight type %d", who, type);
    if (rows < 1 || cols < kSuper || cols % kSuper != 0 || rows > ((int64_t)1 << 30) ||
        cols > ((int64_t)1 << 24))
        return fail(MMQ_E_SHAPE, "%s: rows=%lld cols=%lld (cols must be a multiple of 256)", who,
                    (long long)rows, (long long)cols);
    if (uses & ~(MMQ_USE_GEMM | MMQ_USE_GEMV | MMQ_USE_GEMM_PACKED))
        return fail(MMQ_E_ARG, "%s: unknown uses 0x%x", who, uses);
    if ((uses & MMQ_USE_GEMM_PACKED) && !(uses & MMQ_USE_GEMM))
        return fail(MMQ_E_ARG, "%s: MMQ_USE_GEMM_PACKED needs MMQ_USE_GEMM (uses=%u)", who, uses);
    if ((uses & MMQ_USE_GEMM_PACKED) && type != MMQ_Q4_K)
        return fail(MMQ_E_TYPE, "%s: packed matmul tiles are for q4_K weights only (type %d)", who,
                    type);
    if (uses == 0)
        uses = type == MMQ_Q4_K ? MMQ_USE_GEMM
               : type == MMQ_Q5_K ? MMQ_USE_GEMV : (MMQ_USE_GEMM | MMQ_USE_GEMV);
    if (type == MMQ_Q5_K && (uses & MMQ_USE_GEMM))
        return fail(MMQ_E_TYPE, "%s: q5_K has a one-token GEMV arm only (uses=%u)", who, uses);

    mmq_weight* h = new mmq_weight();
    h->ctx = c;
    h->dry = c->dry;
    WeightDev& w = h->w;
    w.type = type;
    w.rows = rows;
    w.cols = cols;
    w.rows_pad = round_up(rows, kTileO);
    w.uses = uses;
    w.packed = (uses & MMQ_USE_GEMM_PACKED) != 0;
    const int64_t nsb = cols / kSuper, nb = cols / kBlock, og = w.rows_pad / 32;
    const int64_t bpb = type == MMQ_Q4_K ? 144 : type == MMQ_Q5_K ? 176 : 210;
    const int64_t raw_bytes = rows * nsb * bpb;
    // matmul tiles: one f16 per weight (q4_K sc*q, q6_K q-32; packed q4_K:
    // half a byte per weight plus 8 f16 sub-scales per row and superblock),
    // superblock scales, and per (row group, superblock) the q4_K mins or the
    // q6_K sub-scales as f16
    const int64_t wa_b = w.packed ? w.rows_pad * cols / 2 : w.rows_pad * cols * 2;
    const int64_t ws_b = w.packed ? w.rows_pad * nsb * 16 : 0;
    const int64_t dmr_b = og * nsb * (type == MMQ_Q4_K ? 64 : 32) * 4;
    const int64_t mf_b = og * nsb * (type == MMQ_Q4_K ? 512 * 2 : 32 * 16 * 2);
    // one-token GEMV tiles: q6_K ql/qh/sc/d; q4_K nibbles (in ql), (sc, m)
    // pairs (in sc) and (d, dmin) per superblock (in d), no qh; q5_K as
    // q4_K plus the fifth bits (4 B per 32 weights)
    const int64_t ql_b = rows * nb * 16,
                  qh_b = type == MMQ_Q6_K ? rows * nb * 8 : type == MMQ_Q5_K ? rows * nb * 4 : 0,
                  sc_b = rows * nb * 2, dv_b = rows * nsb * (type == MMQ_Q6_K ? 4 : 8);
    // the matmul addresses its tiles with 32-bit buffer offsets
    if ((uses & MMQ_USE_GEMM) && wa_b > (int64_t)0xFFFFFFFF) {
        delete h;
        return fail(MMQ_E_SHAPE, "%s: %lld x %lld needs %lld bytes of matmul tiles (limit 4 GiB); "
                    "register it as several row blocks", who, (long long)rows, (long long)cols,
                    (long long)wa_b);
    }
    int64_t total = 0;
    if (uses & MMQ_USE_GEMM) total += wa_b + ws_b + dmr_b + mf_b;
    if (uses & MMQ_USE_GEMV) total += ql_b + qh_b + sc_b + dv_b;
    w.bytes = total;
    if (c->dry) {
        c->weight_bytes += total;
        *out = h;
        return MMQ_OK;
    }
    int rc = use_device(c);
    if (rc) { delete h; return rc; }

    std::vector<void*> allocs;
    auto cleanup = [&]() {
        for (void* p : allocs) (void)hipFree(p);
        delete h;
    };
    auto dalloc = [&](int64_t bytes, void** p) -> bool {
        if (hipMalloc(p, (size_t)bytes) != hipSuccess) {
            (void)hipGetLastError();
            return false;
        }
        allocs.push_back(*p);
        return true;
    };
    void* raw_dev = nullptr;
    if (!dalloc(raw_bytes, &raw_dev)) { cleanup(); return fail(MMQ_E_OOM, "%s: staging alloc failed", who); }
    hipError_t e = hipMemcpy(raw_dev, raw_host, (size_t)raw_bytes, hipMemcpyHostToDevice);
    if (e != hipSuccess) { cleanup(); return hip_fail(e, "mmq_register_weight: copy"); }
    if (uses & MMQ_USE_GEMM) {
        void *p1 = nullptr, *p2 = nullptr, *p3 = nullptr, *p4 = nullptr;
        if (!dalloc(wa_b, &p1) || !dalloc(dmr_b, &p2) || (mf_b && !dalloc(mf_b, &p3)) ||
            (ws_b && !dalloc(ws_b, &p4))) {
            cleanup();
            return fail(MMQ_E_OOM, "%s: %lld bytes of matmul tiles", who,
                        (long long)(wa_b + ws_b + dmr_b + mf_b));
        }
        w.wa = (_Float16*)p1; w.dmr = (float*)p2; w.mfrag = (_Float16*)p3; w.wsc = (uint4*)p4;
        e = hipMemset(p1, 0, (size_t)wa_b);   // padded rows stay zero weights
        if (e == hipSuccess) e = hipMemset(p2, 0, (size_t)dmr_b);
        if (e == hipSuccess && p3) e = hipMemset(p3, 0, (size_t)mf_b);
        if (e == hipSuccess && p4) e = hipMemset(p4, 0, (size_t)ws_b);
        if (e == hipSuccess) e = launch_repack_gemm((const uint8_t*)raw_dev, w, nullptr);
        if (e != hipSuccess) { cleanup(); return hip_fail(e, "mmq_register_weight: repack"); }
    }
    if (uses & MMQ_USE_GEMV) {
        void *p1 = nullptr, *p2 = nullptr, *p3 = nullptr, *p4 = nullptr;
        if (!dalloc(ql_b, &p1) || (qh_b && !dalloc(qh_b, &p2)) || !dalloc(sc_b, &p3) ||
            !dalloc(dv_b, &p4)) {
            cleanup();
            return fail(MMQ_E_OOM, "%s: GEMV tiles", who);
        }
        w.gv_ql = (uint4*)p1; w.gv_sc = (int16_t*)p3; w.gv_d = (float*)p4;
        if (type == MMQ_Q5_K) w.gv_h5 = (uint32_t*)p2;
        else w.gv_qh = (uint2*)p2;
        e = launch_repack_gemv((const uint8_t*)raw_dev, w, nullptr);
        if (e != hipSuccess) { cleanup(); return hip_fail(e, "mmq_register_weight: repack"); }
    }
    e = hipDeviceSynchronize();
    if (e != hipSuccess) { cleanup(); return hip_fail(e, "mmq_register_weight: sync"); }
    (void)hipFree(raw_dev);
    allocs.erase(allocs.begin());
    c->weight_bytes += total;
    *out = h;
    return MMQ_OK;
}

void mmq_weight_free(mmq_weight* h) {
    if (!h) return;
    if (!h->dry) {
        (void)hipSetDevice(h->ctx->device);
        (void)hipDeviceSynchronize();
        void* ps[] = {h->w.wa,    h->w.dmr,   h->w.mfrag, h->w.wsc,  h->w.gv_ql,
                      h->w.gv_qh, h->w.gv_h5, h->w.gv_sc, h->w.gv_d};
        for (void* p : ps)
            if (p) (void)hipFree(p);
    }
    h->ctx->weight_bytes -= h->w.bytes;
    delete h;
}

int64_t mmq_weight_bytes(const mmq_weight* h) { return h ? h->w.bytes : 0; }

int mmq_quant_rms(mmq_ctx* c, const float* x, const float* w, float* y, int64_t n, int64_t d,
                  float eps, int write_y, void* stream) {
    return produce(c, kProdRms, "mmq_quant_rms", x, w, y, n, d, eps, write_y, stream);
}

int mmq_quant_swiglu(mmq_ctx* c, const float* gate, const float* up, float* y, int64_t n,
                     int64_t d, int write_y, void* stream) {
    return produce(c, kProdSwiglu, "mmq_quant_swiglu", gate, up, y, n, d, 0.0f, write_y, stream);
}

int mmq_quant_f32(mmq_ctx* c, const float* x, int64_t n, int64_t d, void* stream) {
    return produce(c, kProdF32, "mmq_quant_f32", x, nullptr, nullptr, n, d, 0.0f, 0, stream);
}

// Grow-only scratch for K-split partials (counted against the scratch cap
// with the plane slots; never grown during a capture, retired if captured).
static int acquire_part(mmq_ctx* c, int64_t bytes, bool in_capture, const char* who) {
    if (bytes <= c->part_cap) return MMQ_OK;
    if (in_capture)
        return fail(MMQ_E_ARG, "%s: split-K scratch must grow to %lld bytes during stream "
                    "capture; make the same calls once before capturing", who, (long long)bytes);
    const int64_t total = c->plane_bytes - c->part_cap + bytes;
    if (c->cap >= 0 && total > c->cap)
        return fail(MMQ_E_OOM, "%s: scratch cap %lld bytes exceeded by split-K partials", who,
                    (long long)c->cap);
    if (!c->dry) {
        if (c->part && c->captured) c->retired.push_back(c->part);
        else if (c->part) (void)hipFree(c->part);
        c->part = nullptr;
        void* m = nullptr;
        if (hipMalloc(&m, (size_t)bytes) != hipSuccess) {
            (void)hipGetLastError();
            c->plane_bytes -= c->part_cap;
            c->part_cap = 0;
            return fail(MMQ_E_OOM, "%s: hipMalloc of %lld bytes of split-K scratch failed", who,
                        (long long)bytes);
        }
        c->part = m;
    }
    c->plane_bytes += bytes - c->part_cap;
    c->part_cap = bytes;
    return MMQ_OK;
}

// The small-n band: the few-token GEMV serves n <= kSmallN when it needs
// one pass; a second pass (the weights streamed twice) still beats the split
// matmul for n <= 8 (rows too wide for 8 tokens in the LDS: q6_K 3584 x 18944
// at n = 8, 34 against 41 us) and for small weights up to n = 16 (q4_K
// 3584 x 3584 at n = 12-16, 13.7 against 19.2 us), but not for the large FFN
// weights at n = 12-16 (44-64 against 35-40 us).
constexpr int64_t kSmallN = 16;
constexpr int64_t kTwoPassMaxWeights = 16000000;   // rows * cols

static bool small_n_gemv(const WeightDev& w, int64_t n) {
    if (n > kSmallN || !(w.uses & MMQ_USE_GEMV)) return false;
    const int passes = mmvqn_passes(w.cols, n);
    if (passes == 1) return true;
    return passes == 2 && (n <= 8 || w.rows * w.cols <= kTwoPassMaxWeights);
}

static int gemm_common(mmq_ctx* c, const mmq_weight* w, const float* a, int64_t n, float* out,
                       void* stream, int type, const char* who) {
    int rc = consume_check(c, w, a, n, out, type, MMQ_USE_GEMM, who);
    if (rc) return rc;
    // the matmul addresses the plane with 32-bit offsets
    if (round_up(n, kPlaneRows) * w->w.cols >= ((int64_t)1 << 31))
        return fail(MMQ_E_SHAPE, "%s: plane of %lld x %lld codes exceeds 2 GiB; split the tokens",
                    who, (long long)n, (long long)w->w.cols);
    if ((rc = use_device(c))) return rc;
    // The small-n band: with GEMV tiles registered, few tokens run on the
    // dot4 GEMV path (one launch streams the packed weights once for a pass
    // of up to 8 tokens) instead of the 128-token matmul tiles.
    const bool small = small_n_gemv(w->w, n);
    if (small) {
        PlaneView pl;
        if ((rc = plane_for(c, who, a, n, w->w.cols, stream, &pl))) return rc;
        written(c, out, n * w->w.rows * 4);
        if (type == MMQ_Q4_K) c->st.launches_gemm_q4k++;
        else c->st.launches_gemm_q6k++;
        c->st.small_n_gemv++;
        if (c->dry) return MMQ_OK;
        hipStream_t s = (hipStream_t)stream;
        hipError_t e;
        if (n == 1)
            e = type == MMQ_Q4_K ? launch_mmvq_q4k(w->w, pl, out, s) : launch_mmvq_q6k(w->w, pl, out, s);
        else
            e = type == MMQ_Q4_K ? launch_mmvqn_q4k(w->w, pl, n, out, c->n_cu, s)
                                 : launch_mmvqn_q6k(w->w, pl, n, out, c->n_cu, s);
        return after_launch(c, e, s, who);
    }
    const GemmPlan plan = gemm_plan(w->w, n, c->n_cu);
    if (plan.part_floats > 0 &&
        (rc = acquire_part(c, plan.part_floats * 4, capturing(c, (hipStream_t)stream), who)))
        return rc;
    PlaneView pl;
    if ((rc = plane_for(c, who, a, n, w->w.cols, stream, &pl))) return rc;
    written(c, out, n * w->w.rows * 4);
    if (type == MMQ_Q4_K) c->st.launches_gemm_q4k++;
    else c->st.launches_gemm_q6k++;
    if (c->dry) return MMQ_OK;
    hipStream_t s = (hipStream_t)stream;
    return after_launch(c, launch_gemm(w->w, pl, n, out, (float*)c->part, plan, s), s, who);
}

int mmq_gemm_q4k(mmq_ctx* c, const mmq_weight* w, const float* a, int64_t n, float* out,
                 void* stream) {
    return gemm_common(c, w, a, n, out, stream, MMQ_Q4_K, "mmq_gemm_q4k");
}

int mmq_gemm_q6k(mmq_ctx* c, const mmq_weight* w, const float* a, int64_t n, float* out,
                 void* stream) {
    return gemm_common(c, w, a, n, out, stream, MMQ_Q6_K, "mmq_gemm_q6k");
}

int mmvq_q6k(mmq_ctx* c, const mmq_weight* w, const float* a, float* out, void* stream) {
    const char* who = "mmvq_q6k";
    int rc = consume_check(c, w, a, 1, out, MMQ_Q6_K, MMQ_USE_GEMV, who);
    if (rc) return rc;
    if ((rc = use_device(c))) return rc;
    PlaneView pl;
    if ((rc = plane_for(c, who, a, 1, w->w.cols, stream, &pl))) return rc;
    written(c, out, w->w.rows * 4);
    c->st.launches_mmvq_q6k++;
    if (c->dry) return MMQ_OK;
    hipStream_t s = (hipStream_t)stream;
    return after_launch(c, launch_mmvq_q6k(w->w, pl, out, s), s, who);
}

int mmvq_q6k_noalloc(mmq_ctx* c, const mmq_weight* w, const float* a, float* out,
                     void* stream) {
    const char* who = "mmvq_q6k_noalloc";
    int rc = consume_check(c, w, a, 1, out, MMQ_Q6_K, MMQ_USE_GEMV, who);
    if (rc) return rc;
    const int64_t cols = w->w.cols;
    if (cols > kStaticMaxCols)
        return fail(MMQ_E_SHAPE, "%s: cols=%lld exceeds %lld, the one-token plane this call "
                    "holds without allocating", who, (long long)cols, (long long)kStaticMaxCols);
    if ((rc = use_device(c))) return rc;
    if (capturing(c, (hipStream_t)stream)) c->captured = true;
    // a recorded plane serves as in mmvq_q6k; a miss quantises into the static
    // plane and records nothing (no slot is acquired, so nothing can grow)
    PlaneView pl{};
    bool quantise = false;
    const int idx = find_entry(c, a, 1, cols);
    if (idx >= 0) {
        c->st.cache_hits++;
        c->entries[idx].last = ++c->tick;
        if (!c->dry) pl = view_of(c, idx);
    } else {
        if (overlaps_dead(c, a, cols * 4)) return refuse_dead(c, who, a);
        c->st.cache_misses++;
        c->st.launches_quant_f32++;
        quantise = true;
        if (!c->dry) {
            pl.q = (int8_t*)c->static_plane;
            pl.ds = (uint2*)((char*)c->static_plane + kStaticMaxCols);
            pl.rows = 1;   // the GEMV reads row 0 only: no padded rows
            pl.d = cols;
        }
    }
    written(c, out, w->w.rows * 4);
    c->st.launches_mmvq_q6k++;
    if (c->dry) return MMQ_OK;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = hipSuccess;
    if (quantise) e = launch_producer(kProdF32, a, nullptr, nullptr, 1, cols, 0.0f, false, pl, s);
    if (e == hipSuccess) e = launch_mmvq_q6k(w->w, pl, out, s);
    return after_launch(c, e, s, who);
}

int mmvq_q4k(mmq_ctx* c, const mmq_weight* w, const float* a, float* out, void* stream) {
    const char* who = "mmvq_q4k";
    int rc = consume_check(c, w, a, 1, out, MMQ_Q4_K, MMQ_USE_GEMV, who);
    if (rc) return rc;
    if ((rc = use_device(c))) return rc;
    PlaneView pl;
    if ((rc = plane_for(c, who, a, 1, w->w.cols, stream, &pl))) return rc;
    written(c, out, w->w.rows * 4);
    c->st.launches_mmvq_q4k++;
    if (c->dry) return MMQ_OK;
    hipStream_t s = (hipStream_t)stream;
    return after_launch(c, launch_mmvq_q4k(w->w, pl, out, s), s, who);
}

int mmq_gemv_q6k_f32(mmq_ctx* c, const mmq_weight* w, const float* x, float* out,
                     void* stream) {
    const char* who = "mmq_gemv_q6k_f32";
    int rc = consume_check(c, w, x, 1, out, MMQ_Q6_K, MMQ_USE_GEMV, who);
    if (rc) return rc;
    if (w->w.cols > kGemvF32MaxCols)
        return fail(MMQ_E_SHAPE, "%s: cols=%lld exceeds %lld (x is staged whole in LDS)", who,
                    (long long)w->w.cols, (long long)kGemvF32MaxCols);
    // the kernel reads x itself: a buffer a skip-write producer never wrote is refused
    if (overlaps_dead(c, x, w->w.cols * 4)) return refuse_dead(c, who, x);
    if ((rc = use_device(c))) return rc;
    written(c, out, w->w.rows * 4);
    c->st.launches_gemv_f32++;
    if (c->dry) return MMQ_OK;
    hipStream_t s = (hipStream_t)stream;
    return after_launch(c, launch_gemv_f32_q6k(w->w, x, out, s), s, who);
}

int mmq_decode_q6k(mmq_ctx* c, const mmq_weight* w, const float* x, float* out, void* stream) {
    const char* who = "mmq_decode_q6k";
    int rc = consume_check(c, w, x, 1, out, MMQ_Q6_K, MMQ_USE_GEMV, who);
    if (rc) return rc;
    // The f32 path only where it is cheaper (small od*id) and possible: x was
    // written (not a dead key) and has no plane yet (a recorded plane makes
    // the GEMV free of its quantise).
    const int64_t od = w->w.rows, id = w->w.cols;
    if (od * id < MMQ_DECODE_F32_GATE && id <= kGemvF32MaxCols && find_entry(c, x, 1, id) < 0 &&
        !overlaps_dead(c, x, id * 4))
        return mmq_gemv_q6k_f32(c, w, x, out, stream);
    return mmvq_q6k(c, w, x, out, stream);
}

int mmvq_q5k(mmq_ctx* c, const mmq_weight* w, const float* a, float* out, void* stream) {
    const char* who = "mmvq_q5k";
    int rc = consume_check(c, w, a, 1, out, MMQ_Q5_K, MMQ_USE_GEMV, who);
    if (rc) return rc;
    if ((rc = use_device(c))) return rc;
    PlaneView pl;
    if ((rc = plane_for(c, who, a, 1, w->w.cols, stream, &pl))) return rc;
    written(c, out, w->w.rows * 4);
    c->st.launches_mmvq_q5k++;
    if (c->dry) return MMQ_OK;
    hipStream_t s = (hipStream_t)stream;
    return after_launch(c, launch_mmvq_q5k(w->w, pl, out, s), s, who);
}

int mmq_register_foreign_consumer(mmq_ctx* c, int kind) {
    if (!c) return fail(MMQ_E_ARG, "mmq_register_foreign_consumer: null context");
    if (kind != MMQ_FOREIGN_F32 && kind != MMQ_FOREIGN_QUANT)
        return fail(MMQ_E_ARG, "mmq_register_foreign_consumer: unknown kind %d", kind);
    if (c->plane_only)
        fprintf(stderr,
                "libmmq: a consumer that reads f32 activations directly was registered (%s); "
                "skip-write producers now write y as well\n",
                kind == MMQ_FOREIGN_F32 ? "2-D f32 weight" : "weight type without a plane path");
    c->plane_only = false;
    return MMQ_OK;
}

int mmq_plane_only(const mmq_ctx* c) { return c && c->plane_only ? 1 : 0; }

void mmq_cache_clear(mmq_ctx* c) {
    if (!c) return;
    for (Entry& e : c->entries) e.used = false;
    c->dead.clear();
}

int mmq_cache_invalidate(mmq_ctx* c, const void* key) {
    if (!c) return fail(MMQ_E_ARG, "mmq_cache_invalidate: null context");
    for (Entry& e : c->entries)
        if (e.used && e.key == key) e.used = false;
    // every piece of the dead range recorded for key, also the pieces a later
    // partial write left of it
    c->dead.erase(std::remove_if(c->dead.begin(), c->dead.end(),
                                 [&](const DeadRange& r) { return r.key == (uintptr_t)key; }),
                  c->dead.end());
    return MMQ_OK;
}

int mmq_plane_export(mmq_ctx* c, const void* key, int64_t n, int64_t d, int include_pad,
                     int8_t* q, float* dq, int32_t* s, void* stream) {
    const char* who = "mmq_plane_export";
    if (!c || !q || !dq || !s) return fail(MMQ_E_ARG, "%s: null argument", who);
    if ((((uintptr_t)dq) | ((uintptr_t)s)) & 3u)
        return fail(MMQ_E_ARG, "%s: dq and s must be 4-byte aligned", who);
    const int idx = find_entry(c, key, n, d);
    if (idx < 0) return fail(MMQ_E_ARG, "%s: no plane recorded for (%p, %lld, %lld)", who, key,
                             (long long)n, (long long)d);
    if (c->dry) return fail(MMQ_E_DEVICE, "%s: dry-run context holds no planes", who);
    int rc = use_device(c);
    if (rc) return rc;
    const PlaneView pl = view_of(c, idx);
    const int64_t rows = include_pad ? pl.rows : n;
    const int64_t nb = d / kBlock;
    written(c, q, rows * d);
    written(c, dq, rows * nb * 4);
    written(c, s, rows * nb * 4);
    hipStream_t st = (hipStream_t)stream;
    hipError_t e = hipMemcpyAsync(q, pl.q, (size_t)(rows * d), hipMemcpyDeviceToDevice, st);
    if (e == hipSuccess) e = launch_plane_split(pl.ds, dq, s, rows * nb, st);
    return after_launch(c, e, st, who);
}

int mmq_stats(mmq_ctx* c, mmq_stats_t* st) {
    if (!c || !st) return fail(MMQ_E_ARG, "mmq_stats: null argument");
    *st = c->st;
    int64_t live = 0;
    for (const Entry& e : c->entries) live += e.used ? 1 : 0;
    st->cache_entries = live;
    st->plane_bytes = c->plane_bytes;
    st->weight_bytes = c->weight_bytes;
    return MMQ_OK;
}

}  // extern "C"
