// ftm_api.cpp -- the C ABI of libftm (include/ftm.h): argument checks, the
// split-sequence choice, the per-(device, stream) workspace, launches and
// the optional kernel timing.  Host code only; the kernels live in
// decode_attention.hip.
#include "ftm.h"

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <map>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "ftm_internal.hpp"

namespace {

thread_local std::string g_last_error;

int fail(int status, const std::string& msg) {
    g_last_error = msg;
    return status;
}

// ---------------------------------------------------------------------------
// Workspace: one growing buffer per (device, stream).  Reused across calls
// ([lpnh.cn/news/2765398] section 2.2: intermediate buffers are pooled and
// recycled instead of allocated per layer).  A call that needs more
// allocates a larger buffer (at least twice the old one, so the kept
// buffers together stay below the current one) and keeps the old one
// until ftm_release_workspaces: hipFree would wait for the device, and
// work already enqueued, or a captured graph, may still use it.
// ---------------------------------------------------------------------------
struct Workspace {
    void* ptr = nullptr;        // split partials
    size_t bytes = 0;
    int* counters = nullptr;    // per-unit counts of the balanced schedule, zero between calls
    size_t n_counters = 0;
};
std::mutex g_ws_mutex;
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;
// Buffers that larger ones replaced, freed by ftm_release_workspaces.
std::vector<std::pair<int, void*>> g_retired;

// Partials buffer of at least `bytes` and, when n_counters > 0, a counter
// array of at least that many ints, zero when the kernels on `stream`
// reach it, for (device, stream).  Never waits for the device.
int get_workspace(int device, hipStream_t stream, size_t bytes, size_t n_counters, bool capturing,
                  void** out, int** counters) {
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    Workspace& w = g_ws[{device, stream}];
    if (capturing && (w.bytes < bytes || w.n_counters < n_counters))
        return fail(FTM_ERR_INVALID_ARG,
                    "the stream is being captured and its workspace would have to grow: make one "
                    "call of this shape on this stream before capturing");
    if (w.bytes < bytes) {
        const size_t grow = std::max(bytes + bytes / 4, 2 * w.bytes);
        void* np = nullptr;
        hipError_t e = hipMalloc(&np, grow);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return fail(FTM_ERR_OUT_OF_MEMORY, "workspace of " + std::to_string(grow) +
                                                   " bytes: " + hipGetErrorString(e));
        }
        if (w.ptr) g_retired.push_back({device, w.ptr});
        w.ptr = np;
        w.bytes = grow;
    }
    if (w.n_counters < n_counters) {
        const size_t grow = std::max(n_counters + n_counters / 4 + 64, 2 * w.n_counters);
        int* nc = nullptr;
        hipError_t e = hipMalloc(&nc, grow * sizeof(int));
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return fail(FTM_ERR_OUT_OF_MEMORY, std::string("counter array: ") + hipGetErrorString(e));
        }
        // cleared on the call's stream, ahead of the kernel that uses it
        e = ftm::launch_zero_ints(nc, grow, stream);
        if (e != hipSuccess) {
            g_retired.push_back({device, nc});
            return fail(FTM_ERR_HIP, std::string("counter clear: ") + hipGetErrorString(e));
        }
        if (w.counters) g_retired.push_back({device, w.counters});
        w.counters = nc;
        w.n_counters = grow;
    }
    *out = w.ptr;
    if (counters) *counters = w.counters;
    return FTM_OK;
}

// ---------------------------------------------------------------------------
// Kernel timing (measurement only).
// ---------------------------------------------------------------------------
struct Timing {
    bool on = false;
    int capacity = 0;
    std::vector<std::pair<hipEvent_t, hipEvent_t>> ev[2];
    int used[2] = {0, 0};
};
std::mutex g_t_mutex;
Timing g_t;

void destroy_events_locked() {
    for (int k = 0; k < 2; ++k) {
        for (auto& pr : g_t.ev[k]) {
            (void)hipEventDestroy(pr.first);
            (void)hipEventDestroy(pr.second);
        }
        g_t.ev[k].clear();
        g_t.used[k] = 0;
    }
}

// Returns the event pair for the next launch of `kind`, or nulls.
std::pair<hipEvent_t, hipEvent_t> timing_slot(int kind) {
    std::lock_guard<std::mutex> lock(g_t_mutex);
    if (!g_t.on || g_t.used[kind] >= (int)g_t.ev[kind].size()) return {nullptr, nullptr};
    return g_t.ev[kind][g_t.used[kind]++];
}

std::atomic<int> g_split_chunk{0};
std::atomic<int> g_waves{0};

int env_int(const char* name, int dflt) {
    const char* v = std::getenv(name);
    return v && *v ? std::atoi(v) : dflt;
}

ftm::Tuning read_tuning() {
    ftm::Tuning t{};
    t.validate = env_int("FTM_VALIDATE", 0);
    t.waves = env_int("FTM_WAVES", 0);
    t.split_chunk = env_int("FTM_SPLIT_CHUNK", 0);
    t.gqa_valu = env_int("FTM_GQA_VALU", 0);
    t.gqa_blocks_per_cu = env_int("FTM_GQA_BLOCKS_PER_CU", 0);
    t.gqa_unit_cost = env_int("FTM_GQA_UNIT_COST", -1);
    t.gqa_skew_a = t.gqa_skew_b = 0;
    if (const char* e = std::getenv("FTM_GQA_SKEW")) {
        int a = 0, b = 0;
        if (std::sscanf(e, "%d,%d", &a, &b) == 2) {
            t.gqa_skew_a = a;
            t.gqa_skew_b = b;
        }
    }
    t.qkv_column_tiles = env_int("FTM_QKV_COLUMN_TILES", 0);
    t.qkv_k_split = env_int("FTM_QKV_K_SPLIT", -1);
    return t;
}

// The current settings.  A reload publishes a new copy and leaves the old
// one in place (a reader may still hold it; reloads are rare).
std::atomic<const ftm::Tuning*> g_tuning{nullptr};

// Launch shape: waves per workgroup and chunk length.
//
// The kernel is bound by HBM bandwidth, which needs about 64 KiB of loads in
// flight per CU, all CUs busy and equal work per workgroup.  When the
// (sequence, KV head, head group) units are about one per CU, a 16-wave
// workgroup per unit (split only if there are fewer units than CUs) keeps a
// CU full with one launch and no combine.  With many units, 4-wave
// workgroups several to a CU balance better.  Passes over several query
// heads, and INT8 caches, need more registers per wave and take 4 waves.
struct Shape {
    int nw;
    int chunk;
};

Shape choose_shape(int kv, int head_dim, int gtile, int units, int step, int n_cu) {
    int nw = g_waves.load();
    if (nw == 0) nw = ftm::tuning().waves;
    bool short_pass = false;
    if (nw != 4 && nw != 16) {
        nw = (ftm::wide_ok(kv, gtile) && units < 2 * n_cu) ? 16 : 4;
        // a short sequence leaves much of a 16-wave workgroup idle: up to
        // four 4-wave iterations, a 4-wave single pass is shorter (7b layer
        // shape at 128 / 256 / 512 positions: 6.6 / 9.1 / 13.9 against
        // 7.6 / 9.9 / 14.4 us; equal at 768, slower at 1024)
        if (nw == 16 && step <= 4 * ftm::tile_rows(kv, head_dim, gtile, 4)) {
            nw = 4;
            short_pass = true;
        }
    }
    if (nw == 16 && !ftm::wide_ok(kv, gtile)) nw = 4;
    const int tile = ftm::tile_rows(kv, head_dim, gtile, nw);
    int forced = g_split_chunk.load();
    if (forced == 0) forced = ftm::tuning().split_chunk;
    int chunk;
    if (forced > 0) {
        chunk = forced;
    } else if (short_pass) {
        chunk = step;                       // one pass per (b, j): no combine
    } else {
        const long target_blocks = nw == 16 ? n_cu : 4L * n_cu;
        long want_s = (target_blocks + units - 1) / units;
        if (want_s < 1) want_s = 1;
        chunk = (int)((step + want_s - 1) / want_s);
    }
    chunk = (chunk + tile - 1) / tile * tile;
    return {nw, chunk};
}

int cu_count(int device) {
    static std::mutex m;
    static std::map<int, int> cache;
    std::lock_guard<std::mutex> lock(m);
    auto it = cache.find(device);
    if (it != cache.end()) return it->second;
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || n <= 0)
        n = 256;
    cache[device] = n;
    return n;
}

// Validated arguments of one decode step, contiguous or paged.
struct Call {
    const void *q, *k_new, *v_new, *qkv_bias;
    void *k_cache, *v_cache;
    const int32_t* seq_lens;
    int batch, capacity, step, n_heads, n_kv_heads, head_dim, kv_dtype;
    float* kv_scales;
    void* out;
    hipStream_t stream;
    // paged
    const int32_t* block_table;
    int page_shift, max_pages, n_pages;
    // scratch from the library's fixed device array instead of the workspace
    bool static_ws;
};

}  // namespace

const ftm::Tuning& ftm::tuning() {
    const Tuning* t = g_tuning.load(std::memory_order_acquire);
    if (t) return *t;
    const Tuning* fresh = new Tuning(read_tuning());
    const Tuning* expected = nullptr;
    if (g_tuning.compare_exchange_strong(expected, fresh, std::memory_order_acq_rel)) return *fresh;
    delete fresh;
    return *expected;
}

// A captured sequence of calls, instantiated for replay.
struct ftm_graph_s {
    hipGraph_t graph;
    hipGraphExec_t exec;
};

extern "C" {

const char* ftm_version(void) { return "libftm 0.1 (gfx950)"; }

const char* ftm_last_error(void) { return g_last_error.c_str(); }

size_t ftm_kv_cache_bytes(int batch, int n_kv_heads, int max_seq_len, int head_dim, ftm_dtype kv_dtype) {
    if (batch < 1 || n_kv_heads < 1 || max_seq_len < 1 || head_dim < 1) return 0;
    size_t elem;
    switch (kv_dtype) {
    case FTM_F32: elem = 4; break;
    case FTM_F16:
    case FTM_BF16: elem = 2; break;
    case FTM_I8: elem = 1; break;
    default: return 0;
    }
    const size_t rows = (size_t)batch * n_kv_heads * max_seq_len;
    return 2 * rows * ((size_t)head_dim * elem + (kv_dtype == FTM_I8 ? 4 : 0));
}

int ftm_set_split_chunk(int positions) {
    if (positions < 0) return -1;
    return g_split_chunk.exchange(positions);
}

int ftm_set_workgroup_waves(int waves) {
    if (waves != 0 && waves != 4 && waves != 16) return -1;
    return g_waves.exchange(waves);
}

void ftm_release_workspaces(void) {
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    std::vector<std::pair<int, void*>> all;
    all.swap(g_retired);
    for (auto& kv : g_ws) {
        if (kv.second.ptr) all.push_back({kv.first.first, kv.second.ptr});
        if (kv.second.counters) all.push_back({kv.first.first, kv.second.counters});
    }
    g_ws.clear();
    int cur = 0;
    (void)hipGetDevice(&cur);
    for (auto& r : all) {
        (void)hipSetDevice(r.first);
        (void)hipFree(r.second);
    }
    (void)hipSetDevice(cur);
}

void ftm_tuning_reload(void) {
    g_tuning.store(new ftm::Tuning(read_tuning()), std::memory_order_release);
}

int ftm_timing_enable(int capacity) {
    if (capacity < 1) return fail(FTM_ERR_INVALID_ARG, "timing capacity must be >= 1");
    std::lock_guard<std::mutex> lock(g_t_mutex);
    destroy_events_locked();
    for (int k = 0; k < 2; ++k) {
        g_t.ev[k].reserve(capacity);
        for (int i = 0; i < capacity; ++i) {
            hipEvent_t a, b;
            if (hipEventCreate(&a) != hipSuccess) return fail(FTM_ERR_HIP, "hipEventCreate failed");
            if (hipEventCreate(&b) != hipSuccess) {
                (void)hipEventDestroy(a);
                return fail(FTM_ERR_HIP, "hipEventCreate failed");
            }
            g_t.ev[k].push_back({a, b});
        }
    }
    g_t.capacity = capacity;
    g_t.on = true;
    return FTM_OK;
}

int ftm_timing_disable(void) {
    std::lock_guard<std::mutex> lock(g_t_mutex);
    g_t.on = false;
    destroy_events_locked();
    return FTM_OK;
}

int ftm_timing_read(int kind, int* launches, double* total_ms) {
    if (kind < 0 || kind > 1 || !launches || !total_ms)
        return fail(FTM_ERR_INVALID_ARG, "ftm_timing_read: bad arguments");
    std::lock_guard<std::mutex> lock(g_t_mutex);
    double total = 0.0;
    const int n = g_t.used[kind];
    for (int i = 0; i < n; ++i) {
        auto& pr = g_t.ev[kind][i];
        hipError_t e = hipEventSynchronize(pr.second);
        if (e != hipSuccess) return fail(FTM_ERR_HIP, std::string("hipEventSynchronize: ") + hipGetErrorString(e));
        float ms = 0.0f;
        e = hipEventElapsedTime(&ms, pr.first, pr.second);
        if (e != hipSuccess) return fail(FTM_ERR_HIP, std::string("hipEventElapsedTime: ") + hipGetErrorString(e));
        total += ms;
    }
    g_t.used[kind] = 0;
    *launches = n;
    *total_ms = total;
    return FTM_OK;
}

}  // extern "C"

namespace {

// Checks shared by both layouts; nothing is enqueued on failure.
int check_common(const void* q, const void* k_new, const void* v_new, const void* qkv_bias,
                 const void* k_cache, const void* v_cache, const int32_t* seq_lens, int batch,
                 int capacity, int step, int n_heads, int n_kv_heads, int head_dim, int kv_dtype,
                 const float* kv_scales, const void* out, const char* capacity_name) {
    if (!q || !k_new || !v_new || !k_cache || !v_cache || !out)
        return fail(FTM_ERR_INVALID_ARG, "a required pointer (q, k_new, v_new, k_cache, v_cache, out) is NULL");
    if (batch < 1 || n_heads < 1 || n_kv_heads < 1 || head_dim < 1)
        return fail(FTM_ERR_INVALID_ARG, "batch, n_heads, n_kv_heads and head_dim must be >= 1");
    if (n_heads % n_kv_heads != 0)
        return fail(FTM_ERR_INVALID_ARG, "n_heads (" + std::to_string(n_heads) +
                                             ") is not a multiple of n_kv_heads (" +
                                             std::to_string(n_kv_heads) + ")");
    if (step < 1 || step > capacity)
        return fail(FTM_ERR_INVALID_ARG, "step " + std::to_string(step) + " outside [1, " + capacity_name +
                                             "=" + std::to_string(capacity) + "]");
    if (kv_dtype < FTM_F32 || kv_dtype > FTM_I8)
        return fail(FTM_ERR_INVALID_ARG, "unknown kv_dtype " + std::to_string(kv_dtype));
    if ((kv_dtype == FTM_I8) != (kv_scales != nullptr))
        return fail(FTM_ERR_INVALID_ARG, kv_dtype == FTM_I8 ? "an INT8 cache needs kv_scales"
                                                             : "kv_scales is only for an INT8 cache");
    {
        const void* vec[] = {q, k_new, v_new, qkv_bias, k_cache, v_cache, out};
        for (const void* v : vec)
            if (((uintptr_t)v & 15u) != 0)
                return fail(FTM_ERR_INVALID_ARG, "q, k_new, v_new, qkv_bias, k_cache, v_cache and out must be 16-byte aligned");
        if (((uintptr_t)seq_lens & 3u) != 0 || ((uintptr_t)kv_scales & 3u) != 0)
            return fail(FTM_ERR_INVALID_ARG, "seq_lens and kv_scales must be 4-byte aligned");
    }
    if (head_dim != 64 && head_dim != 128)
        return fail(FTM_ERR_UNSUPPORTED, "head_dim " + std::to_string(head_dim) + " (built: 64, 128)");
    const int G = n_heads / n_kv_heads;
    const int gtile = ftm::group_tile(G);
    const int n_hg = (G + gtile - 1) / gtile;
    if ((long)n_kv_heads * n_hg > 65535 || batch > 65535)
        return fail(FTM_ERR_UNSUPPORTED, "grid too large: n_kv_heads * head groups and batch must be <= 65535");
    return FTM_OK;
}

size_t elem_bytes(int kv_dtype) { return kv_dtype == FTM_F32 ? 4 : (kv_dtype == FTM_I8 ? 1 : 2); }

int decode_impl(const Call& a) {
    hipStream_t stream = a.stream;
    int device = 0;
    hipError_t he = hipGetDevice(&device);
    if (he != hipSuccess) return fail(FTM_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(he));
    // under stream capture nothing may allocate, synchronise or record
    // timing events: the workspace must already be large enough
    bool capturing = false;
    if (stream) {
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        he = hipStreamIsCapturing(stream, &cs);
        if (he != hipSuccess) return fail(FTM_ERR_HIP, std::string("hipStreamIsCapturing: ") + hipGetErrorString(he));
        capturing = cs != hipStreamCaptureStatusNone;
    }

    if (ftm::tuning().validate && a.seq_lens) {
        if (capturing)
            return fail(FTM_ERR_INVALID_ARG, "FTM_VALIDATE reads seq_lens on the host and cannot run under stream capture");
        std::vector<int32_t> h(a.batch);
        he = hipMemcpyAsync(h.data(), a.seq_lens, sizeof(int32_t) * a.batch, hipMemcpyDeviceToHost, stream);
        if (he == hipSuccess) he = hipStreamSynchronize(stream);
        if (he != hipSuccess) return fail(FTM_ERR_HIP, std::string("FTM_VALIDATE copy: ") + hipGetErrorString(he));
        for (int b = 0; b < a.batch; ++b)
            if (h[b] < 1 || h[b] > a.step)
                return fail(FTM_ERR_INVALID_ARG, "seq_lens[" + std::to_string(b) + "] = " +
                                                     std::to_string(h[b]) + " outside [1, step]");
    }

    const int G = a.n_heads / a.n_kv_heads;
    const int gtile = ftm::group_tile(G);
    const int n_hg = (G + gtile - 1) / gtile;
    ftm::Params p{};
    p.q = a.q;
    p.k_new = a.k_new;
    p.v_new = a.v_new;
    p.bias = a.qkv_bias;
    p.k_cache = a.k_cache;
    p.v_cache = a.v_cache;
    p.seq_lens = a.seq_lens;
    p.kv_scales = a.kv_scales;
    p.out = a.out;
    p.B = a.batch;
    p.Lmax = a.capacity;
    p.step = a.step;
    p.H = a.n_heads;
    p.Hkv = a.n_kv_heads;
    p.G = G;
    p.n_hg = n_hg;
    p.qscale = (float)(1.4426950408889634 / std::sqrt((double)a.head_dim));
    p.block_table = a.block_table;
    p.page_shift = a.page_shift;
    p.max_pages = a.max_pages;
    p.n_pages = a.n_pages;

    const int kv_dtype = a.kv_dtype, head_dim = a.head_dim;
    const int units = a.batch * a.n_kv_heads * n_hg;
    // the range schedule counts tiles (units x (tiles + charge)) in 32-bit
    // integers: well inside that range, or the vector pass takes the step
    const int unit_cost = ftm::gqa_unit_cost();
    const int max_tiles = std::max(1, (a.step + 14) / 16);
    const bool balanced = ftm::use_gqa_mfma(kv_dtype, gtile, a.batch) &&
                          (long long)a.batch * a.step * a.n_kv_heads * n_hg < (1LL << 31) &&
                          (long long)units * (max_tiles + unit_cost) < (1LL << 30);
    Shape shape{4, 0};
    p.balanced = balanced;
    if (balanced) {
        // grouped heads on the matrix cores: equal ranges of the units' tiles,
        // one workgroup per CU (and at least one per sequence, which checks
        // that sequence's length); two partial slots per workgroup, merged
        // in the same launch
        p.S = std::max(cu_count(device) * ftm::gqa_blocks_per_cu(), a.batch);
        p.chunk = 0;
        p.direct = 0;
        p.unit_cost = unit_cost;
        ftm::gqa_skew(p.skew_a, p.skew_b);
        // ranges of at least 16 tiles, and long enough that no unit is cut
        // into more than kGqaMaxPieces pieces
        p.range_min = std::max(std::max(16, p.unit_cost + 1),
                               (max_tiles + ftm::kGqaMaxPieces - 3) / (ftm::kGqaMaxPieces - 2));
        const size_t slots = (size_t)2 * p.S * gtile;
        const size_t need = slots * (head_dim + 2) * sizeof(float);
        void* ws = nullptr;
        if (a.static_ws) {
            if (need > ftm::kStaticPartialBytes || (size_t)units > ftm::kStaticCounterInts)
                return fail(FTM_ERR_UNSUPPORTED,
                            "the grouped-query pass needs " + std::to_string(need) + " bytes of partials and " +
                                std::to_string(units) + " counters; the fixed scratch holds " +
                                std::to_string(ftm::kStaticPartialBytes) + " bytes and " +
                                std::to_string(ftm::kStaticCounterInts) + " counters");
            void* scratch = nullptr;
            he = ftm::static_scratch(device, stream, &scratch);
            if (he != hipSuccess) return fail(FTM_ERR_HIP, std::string("scratch set-up: ") + hipGetErrorString(he));
            p.counters = (int*)scratch;
            ws = (char*)scratch + ftm::kStaticCounterInts * sizeof(int);
        } else {
            int st = get_workspace(device, stream, need, units, capturing, &ws, &p.counters);
            if (st != FTM_OK) return st;
        }
        p.ws_o = (float*)ws;
        p.ws_ml = p.ws_o + slots * head_dim;
    } else {
        shape = choose_shape(kv_dtype, head_dim, gtile, units, a.step, cu_count(device));
        p.chunk = shape.chunk;
        p.S = (a.step + p.chunk - 1) / p.chunk;
        p.direct = p.S == 1;
        if (!p.direct) {
            const size_t n_part = (size_t)a.batch * a.n_heads * p.S;
            const size_t need = n_part * (head_dim + 2) * sizeof(float);
            void* ws = nullptr;
            if (a.static_ws) {
                if (need > ftm::kStaticPartialBytes)
                    return fail(FTM_ERR_UNSUPPORTED,
                                "the split pass needs " + std::to_string(need) +
                                    " bytes of partials; the fixed scratch holds " +
                                    std::to_string(ftm::kStaticPartialBytes));
                void* scratch = nullptr;
                he = ftm::static_scratch(device, stream, &scratch);
                if (he != hipSuccess)
                    return fail(FTM_ERR_HIP, std::string("scratch set-up: ") + hipGetErrorString(he));
                ws = (char*)scratch + ftm::kStaticCounterInts * sizeof(int);
            } else {
                int st = get_workspace(device, stream, need, 0, capturing, &ws, nullptr);
                if (st != FTM_OK) return st;
            }
            p.ws_o = (float*)ws;
            p.ws_ml = p.ws_o + n_part * head_dim;
        }
    }

    auto ev = capturing ? std::pair<hipEvent_t, hipEvent_t>{nullptr, nullptr} : timing_slot(0);
    if (ev.first) (void)hipEventRecord(ev.first, stream);
    he = ftm::launch_attention(p, kv_dtype, head_dim, gtile, shape.nw, stream);
    if (ev.second) (void)hipEventRecord(ev.second, stream);
    if (he != hipSuccess) return fail(FTM_ERR_HIP, std::string("attention launch: ") + hipGetErrorString(he));
    if (!balanced && !p.direct) {
        auto ev2 = capturing ? std::pair<hipEvent_t, hipEvent_t>{nullptr, nullptr} : timing_slot(1);
        if (ev2.first) (void)hipEventRecord(ev2.first, stream);
        he = ftm::launch_combine(p, kv_dtype, head_dim, stream);
        if (ev2.second) (void)hipEventRecord(ev2.second, stream);
        if (he != hipSuccess) return fail(FTM_ERR_HIP, std::string("combine launch: ") + hipGetErrorString(he));
    }
    g_last_error.clear();
    return FTM_OK;
}

}  // namespace

extern "C" {

int ftm_decode_mha(const void* q, const void* k_new, const void* v_new, const void* qkv_bias,
                   void* k_cache, void* v_cache, const int32_t* seq_lens, int batch,
                   int max_seq_len, int step, int n_heads, int n_kv_heads, int head_dim,
                   ftm_dtype kv_dtype, float* kv_scales, void* out, hipStream_t stream_ptr) {
    if (max_seq_len < 1) return fail(FTM_ERR_INVALID_ARG, "max_seq_len must be >= 1");
    int st = check_common(q, k_new, v_new, qkv_bias, k_cache, v_cache, seq_lens, batch, max_seq_len,
                          step, n_heads, n_kv_heads, head_dim, kv_dtype, kv_scales, out, "max_seq_len");
    if (st != FTM_OK) return st;
    if ((size_t)max_seq_len * head_dim * elem_bytes(kv_dtype) > 0x7fffffffu)
        return fail(FTM_ERR_UNSUPPORTED, "one (sequence, KV head) cache slab must stay below 2 GiB");
    Call a{q, k_new, v_new, qkv_bias, k_cache, v_cache, seq_lens, batch, max_seq_len, step, n_heads,
           n_kv_heads, head_dim, kv_dtype, kv_scales, out, (hipStream_t)stream_ptr, nullptr, 0, 0, 0, false};
    return decode_impl(a);
}

int ftm_decode_mha_static(const void* q, const void* k_new, const void* v_new, const void* qkv_bias,
                          void* k_cache, void* v_cache, const int32_t* seq_lens, int batch,
                          int max_seq_len, int step, int n_heads, int n_kv_heads, int head_dim,
                          ftm_dtype kv_dtype, float* kv_scales, void* out, hipStream_t stream_ptr) {
    if (max_seq_len < 1) return fail(FTM_ERR_INVALID_ARG, "max_seq_len must be >= 1");
    int st = check_common(q, k_new, v_new, qkv_bias, k_cache, v_cache, seq_lens, batch, max_seq_len,
                          step, n_heads, n_kv_heads, head_dim, kv_dtype, kv_scales, out, "max_seq_len");
    if (st != FTM_OK) return st;
    if ((size_t)max_seq_len * head_dim * elem_bytes(kv_dtype) > 0x7fffffffu)
        return fail(FTM_ERR_UNSUPPORTED, "one (sequence, KV head) cache slab must stay below 2 GiB");
    Call a{q, k_new, v_new, qkv_bias, k_cache, v_cache, seq_lens, batch, max_seq_len, step, n_heads,
           n_kv_heads, head_dim, kv_dtype, kv_scales, out, stream_ptr, nullptr, 0, 0, 0, true};
    return decode_impl(a);
}

int ftm_decode_mha_paged(const void* q, const void* k_new, const void* v_new, const void* qkv_bias,
                         void* k_pages, void* v_pages, const int32_t* block_table, int n_pages,
                         int page_size, int max_pages_per_seq, const int32_t* seq_lens, int batch,
                         int step, int n_heads, int n_kv_heads, int head_dim, ftm_dtype kv_dtype,
                         float* kv_scales, void* out, hipStream_t stream_ptr) {
    if (!block_table) return fail(FTM_ERR_INVALID_ARG, "block_table is NULL");
    if (((uintptr_t)block_table & 3u) != 0) return fail(FTM_ERR_INVALID_ARG, "block_table must be 4-byte aligned");
    if (n_pages < 1 || max_pages_per_seq < 1)
        return fail(FTM_ERR_INVALID_ARG, "n_pages and max_pages_per_seq must be >= 1");
    if (page_size < 16 || page_size > (1 << 16) || (page_size & (page_size - 1)) != 0)
        return fail(FTM_ERR_INVALID_ARG, "page_size " + std::to_string(page_size) +
                                             " must be a power of two in [16, 65536]");
    const long long cap = (long long)max_pages_per_seq * page_size;
    if (cap > 0x7fffffffLL)
        return fail(FTM_ERR_UNSUPPORTED, "max_pages_per_seq * page_size must stay below 2^31");
    int st = check_common(q, k_new, v_new, qkv_bias, k_pages, v_pages, seq_lens, batch, (int)cap, step,
                          n_heads, n_kv_heads, head_dim, kv_dtype, kv_scales, out,
                          "max_pages_per_seq * page_size");
    if (st != FTM_OK) return st;
    int shift = 0;
    while ((1 << shift) < page_size) ++shift;
    Call a{q, k_new, v_new, qkv_bias, k_pages, v_pages, seq_lens, batch, (int)cap, step, n_heads,
           n_kv_heads, head_dim, kv_dtype, kv_scales, out, (hipStream_t)stream_ptr, block_table, shift,
           max_pages_per_seq, n_pages, false};
    return decode_impl(a);
}

int ftm_qkv_proj(const void* x, const void* w, const void* bias, void* q, void* k_new, void* v_new,
                 int batch, int hidden, int n_heads, int n_kv_heads, int head_dim, ftm_dtype act_dtype,
                 hipStream_t stream_ptr) {
    if (!x || !w || !q || !k_new || !v_new)
        return fail(FTM_ERR_INVALID_ARG, "a required pointer (x, w, q, k_new, v_new) is NULL");
    if (batch < 1 || hidden < 1 || n_heads < 1 || n_kv_heads < 1 || head_dim < 1)
        return fail(FTM_ERR_INVALID_ARG, "batch, hidden, n_heads, n_kv_heads and head_dim must be >= 1");
    if (n_heads % n_kv_heads != 0)
        return fail(FTM_ERR_INVALID_ARG, "n_heads (" + std::to_string(n_heads) +
                                             ") is not a multiple of n_kv_heads (" +
                                             std::to_string(n_kv_heads) + ")");
    if (act_dtype != FTM_F16 && act_dtype != FTM_BF16)
        return fail(act_dtype == FTM_F32 ? FTM_ERR_UNSUPPORTED : FTM_ERR_INVALID_ARG,
                    "the projection takes fp16 or bf16 activations and weights, not dtype " +
                        std::to_string(act_dtype));
    {
        const void* vec[] = {x, w, bias, q, k_new, v_new};
        for (const void* v : vec)
            if (((uintptr_t)v & 15u) != 0)
                return fail(FTM_ERR_INVALID_ARG, "x, w, bias, q, k_new and v_new must be 16-byte aligned");
    }
    if (batch > 64)
        return fail(FTM_ERR_UNSUPPORTED, "batch " + std::to_string(batch) + " (built: up to 64 rows)");
    if (hidden % 256 != 0 || hidden > 65536)
        return fail(FTM_ERR_UNSUPPORTED, "hidden " + std::to_string(hidden) +
                                             " (built: multiples of 256 up to 65536)");
    if (head_dim % 16 != 0)
        return fail(FTM_ERR_UNSUPPORTED, "head_dim " + std::to_string(head_dim) + " (built: multiples of 16)");
    const long long n_out = (long long)(n_heads + 2 * n_kv_heads) * head_dim;
    if (n_out / 16 > 0x7fffffffLL || n_out * hidden * 2 > (1LL << 40))
        return fail(FTM_ERR_UNSUPPORTED, "weight matrix too large");
    ftm::QkvParams p{x, w, bias, q, k_new, v_new, batch, hidden, n_heads, n_kv_heads, head_dim, nullptr, nullptr};
    int device = 0;
    hipError_t he = hipGetDevice(&device);
    if (he != hipSuccess) return fail(FTM_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(he));
    const int n_cu = cu_count(device);
    size_t n_counters = 0;
    const size_t need = ftm::qkv_split_workspace(p, n_cu, &n_counters);
    if (need > 0) {
        // the k-split partial sums: the stream's workspace, which under
        // capture must already be large enough
        bool capturing = false;
        if (stream_ptr) {
            hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
            he = hipStreamIsCapturing(stream_ptr, &cs);
            if (he != hipSuccess)
                return fail(FTM_ERR_HIP, std::string("hipStreamIsCapturing: ") + hipGetErrorString(he));
            capturing = cs != hipStreamCaptureStatusNone;
        }
        void* ws = nullptr;
        int st = get_workspace(device, stream_ptr, need, n_counters, capturing, &ws, &p.counters);
        if (st != FTM_OK) return st;
        p.ws = (float*)ws;
    }
    he = ftm::launch_qkv_proj(p, act_dtype, n_cu, (hipStream_t)stream_ptr);
    if (he != hipSuccess) return fail(FTM_ERR_HIP, std::string("projection launch: ") + hipGetErrorString(he));
    g_last_error.clear();
    return FTM_OK;
}

}  // extern "C"

namespace {

// Shared by the contiguous and the paged prefill: cache_rows is max_seq_len
// (contiguous) or max_pages_per_seq * page_size (paged), the rows a sequence
// can hold; block_table null for the contiguous cache.
int prefill_impl(const void* q, const void* k_new, const void* v_new, const void* qkv_bias, void* k_cache,
                 void* v_cache, const int32_t* seq_lens, int batch, int cache_rows, const char* cache_rows_name,
                 int prompt_len, int n_heads, int n_kv_heads, int head_dim, int kv_dtype, float* kv_scales,
                 void* out, void* stream_ptr, const int32_t* block_table, int page_shift, int max_pages,
                 int n_pages) {
    if (!q || !k_new || !v_new || !k_cache || !v_cache || !out)
        return fail(FTM_ERR_INVALID_ARG, "a required pointer (q, k_new, v_new, k_cache, v_cache, out) is NULL");
    if (batch < 1 || cache_rows < 1 || n_heads < 1 || n_kv_heads < 1 || head_dim < 1)
        return fail(FTM_ERR_INVALID_ARG, std::string("batch, ") + cache_rows_name +
                                             ", n_heads, n_kv_heads and head_dim must be >= 1");
    if (n_heads % n_kv_heads != 0)
        return fail(FTM_ERR_INVALID_ARG, "n_heads (" + std::to_string(n_heads) +
                                             ") is not a multiple of n_kv_heads (" +
                                             std::to_string(n_kv_heads) + ")");
    if (prompt_len < 1 || prompt_len > cache_rows)
        return fail(FTM_ERR_INVALID_ARG, "prompt_len " + std::to_string(prompt_len) + " outside [1, " +
                                             cache_rows_name + "=" + std::to_string(cache_rows) + "]");
    if (kv_dtype < FTM_F32 || kv_dtype > FTM_I8)
        return fail(FTM_ERR_INVALID_ARG, "unknown kv_dtype " + std::to_string(kv_dtype));
    if (kv_dtype == FTM_F32) return fail(FTM_ERR_UNSUPPORTED, "prefill takes fp16, bf16 or INT8 caches");
    const bool i8 = kv_dtype == FTM_I8;
    if (i8 != (kv_scales != nullptr))
        return fail(FTM_ERR_INVALID_ARG, "kv_scales must be given for an INT8 cache and only then");
    if (((uintptr_t)kv_scales & 3u) != 0) return fail(FTM_ERR_INVALID_ARG, "kv_scales must be 4-byte aligned");
    {
        const void* vec[] = {q, k_new, v_new, qkv_bias, k_cache, v_cache, out};
        for (const void* v : vec)
            if (((uintptr_t)v & 15u) != 0)
                return fail(FTM_ERR_INVALID_ARG, "q, k_new, v_new, qkv_bias, k_cache, v_cache and out must be 16-byte aligned");
        if (((uintptr_t)seq_lens & 3u) != 0)
            return fail(FTM_ERR_INVALID_ARG, "seq_lens must be 4-byte aligned");
    }
    if (head_dim != 64 && head_dim != 128)
        return fail(FTM_ERR_UNSUPPORTED, "head_dim " + std::to_string(head_dim) + " (built: 64, 128)");
    if (batch > 65535 || (long long)batch * n_heads > 0x7fffffffLL || (prompt_len + 127) / 128 > 65535 ||
        n_kv_heads > 65535 * 16)
        return fail(FTM_ERR_UNSUPPORTED, "grid too large: batch <= 65535, batch * n_heads < 2^31, "
                                         "prompt_len <= 65535 * 128 and n_kv_heads <= 65535 * 16");
    if ((size_t)((prompt_len * (size_t)head_dim + 2047) / 2048) * n_kv_heads > 0x7fffffffu)
        return fail(FTM_ERR_UNSUPPORTED, "prompt_len * head_dim / 2048 * n_kv_heads (append blocks) must stay below 2^31");
    if (!block_table && (size_t)cache_rows * head_dim * 2 > 0x7fffffffu)
        return fail(FTM_ERR_UNSUPPORTED, "one (sequence, KV head) cache slab must stay below 2 GiB");
    if (i8 && ((size_t)prompt_len * head_dim * 2 > 0x7fffffffu ||
               (size_t)prompt_len * n_kv_heads * (head_dim / 16) > 0x7fffffffu))
        return fail(FTM_ERR_UNSUPPORTED, "INT8 prefill: prompt_len * head_dim * 2 bytes (one staged slab) and "
                                         "prompt_len * n_kv_heads * head_dim / 16 must stay below 2^31");
    ftm::PrefillParams p{q, k_new, v_new, qkv_bias, k_cache, v_cache, seq_lens, out, batch, prompt_len,
                         cache_rows, n_heads, n_kv_heads,
                         (float)(1.4426950408889634 / std::sqrt((double)head_dim)),
                         block_table, page_shift, max_pages, n_pages,
                         kv_scales, nullptr, nullptr, nullptr, nullptr, nullptr};
    hipStream_t stream = (hipStream_t)stream_ptr;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (stream && hipStreamIsCapturing(stream, &cs) != hipSuccess)
        return fail(FTM_ERR_HIP, "hipStreamIsCapturing failed");
    const bool capturing = cs != hipStreamCaptureStatusNone;
    // the stream's workspace: over an INT8 cache the staging the attention
    // reads (codes as fp16 and scales, K and V); over a float cache with a
    // bias the bias terms b_q . k of every prompt row and query head
    const size_t rows = (size_t)batch * n_kv_heads * prompt_len;
    const size_t code_bytes = rows * head_dim * 2;
    const size_t stage_bytes = i8 ? 2 * code_bytes + 2 * rows * sizeof(float) : 0;
    const size_t bterm_bytes = !i8 && qkv_bias ? (size_t)batch * n_heads * prompt_len * sizeof(float) : 0;
    if (stage_bytes + bterm_bytes > 0) {
        int device = 0;
        hipError_t e = hipGetDevice(&device);
        if (e != hipSuccess) return fail(FTM_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
        void* ws = nullptr;
        int st = get_workspace(device, stream, stage_bytes + bterm_bytes, 0, capturing, &ws, nullptr);
        if (st != FTM_OK) return st;
        if (i8) {
            p.stage_k = ws;
            p.stage_v = (char*)ws + code_bytes;
            p.stage_ks = (float*)((char*)ws + 2 * code_bytes);
            p.stage_vs = p.stage_ks + rows;
        } else {
            p.bterm = (float*)ws;
        }
    }
    const auto none = std::pair<hipEvent_t, hipEvent_t>{nullptr, nullptr};
    auto ev = capturing ? none : timing_slot(1);
    if (ev.first) (void)hipEventRecord(ev.first, stream);
    hipError_t he = i8 ? ftm::launch_prefill_append_i8(p, head_dim, stream)
                       : ftm::launch_prefill_append(p, kv_dtype, head_dim, stream);
    if (ev.second) (void)hipEventRecord(ev.second, stream);
    if (he != hipSuccess) return fail(FTM_ERR_HIP, std::string("prefill append launch: ") + hipGetErrorString(he));
    ev = capturing ? none : timing_slot(0);
    if (ev.first) (void)hipEventRecord(ev.first, stream);
    he = i8 ? ftm::launch_prefill_attention_i8(p, head_dim, stream)
            : ftm::launch_prefill_attention(p, kv_dtype, head_dim, stream);
    if (ev.second) (void)hipEventRecord(ev.second, stream);
    if (he != hipSuccess) return fail(FTM_ERR_HIP, std::string("prefill attention launch: ") + hipGetErrorString(he));
    g_last_error.clear();
    return FTM_OK;
}

}  // namespace

extern "C" {

int ftm_prefill_mha(const void* q, const void* k_new, const void* v_new, const void* qkv_bias,
                    void* k_cache, void* v_cache, const int32_t* seq_lens, int batch, int max_seq_len,
                    int prompt_len, int n_heads, int n_kv_heads, int head_dim, ftm_dtype kv_dtype,
                    float* kv_scales, void* out, hipStream_t stream_ptr) {
    return prefill_impl(q, k_new, v_new, qkv_bias, k_cache, v_cache, seq_lens, batch, max_seq_len, "max_seq_len",
                        prompt_len, n_heads, n_kv_heads, head_dim, kv_dtype, kv_scales, out, stream_ptr, nullptr, 0,
                        0, 0);
}

int ftm_prefill_mha_paged(const void* q, const void* k_new, const void* v_new, const void* qkv_bias,
                          void* k_pages, void* v_pages, const int32_t* block_table, int n_pages, int page_size,
                          int max_pages_per_seq, const int32_t* seq_lens, int batch, int prompt_len, int n_heads,
                          int n_kv_heads, int head_dim, ftm_dtype kv_dtype, float* kv_scales, void* out,
                          hipStream_t stream_ptr) {
    if (!block_table) return fail(FTM_ERR_INVALID_ARG, "block_table is NULL");
    if (((uintptr_t)block_table & 3u) != 0) return fail(FTM_ERR_INVALID_ARG, "block_table must be 4-byte aligned");
    if (n_pages < 1 || max_pages_per_seq < 1)
        return fail(FTM_ERR_INVALID_ARG, "n_pages and max_pages_per_seq must be >= 1");
    if (page_size < 16 || page_size > (1 << 16) || (page_size & (page_size - 1)) != 0)
        return fail(FTM_ERR_INVALID_ARG, "page_size " + std::to_string(page_size) +
                                             " must be a power of two in [16, 65536]");
    const long long cap = (long long)max_pages_per_seq * page_size;
    if (cap > 0x7fffffffLL)
        return fail(FTM_ERR_UNSUPPORTED, "max_pages_per_seq * page_size must stay below 2^31");
    if ((long long)page_size * head_dim * 2 > 0x7fffffffLL)
        return fail(FTM_ERR_UNSUPPORTED, "one page of one KV head must stay below 2 GiB");
    int shift = 0;
    while ((1 << shift) < page_size) ++shift;
    return prefill_impl(q, k_new, v_new, qkv_bias, k_pages, v_pages, seq_lens, batch, (int)cap,
                        "max_pages_per_seq * page_size", prompt_len, n_heads, n_kv_heads, head_dim, kv_dtype,
                        kv_scales, out, stream_ptr, block_table, shift, max_pages_per_seq, n_pages);
}

int ftm_graph_begin(hipStream_t stream) {
    if (!stream) return fail(FTM_ERR_INVALID_ARG, "the null stream cannot be captured: pass a created stream");
    hipError_t e = hipStreamBeginCapture((hipStream_t)stream, hipStreamCaptureModeThreadLocal);
    if (e != hipSuccess) return fail(FTM_ERR_HIP, std::string("hipStreamBeginCapture: ") + hipGetErrorString(e));
    g_last_error.clear();
    return FTM_OK;
}

int ftm_graph_end(hipStream_t stream, ftm_graph* graph) {
    if (!stream || !graph) return fail(FTM_ERR_INVALID_ARG, "ftm_graph_end: stream and graph must be non-NULL");
    *graph = nullptr;
    hipGraph_t g = nullptr;
    hipError_t e = hipStreamEndCapture((hipStream_t)stream, &g);
    if (e != hipSuccess) {
        if (g) (void)hipGraphDestroy(g);
        return fail(FTM_ERR_HIP, std::string("hipStreamEndCapture: ") + hipGetErrorString(e));
    }
    hipGraphExec_t x = nullptr;
    e = hipGraphInstantiate(&x, g, nullptr, nullptr, 0);
    if (e != hipSuccess) {
        (void)hipGraphDestroy(g);
        return fail(FTM_ERR_HIP, std::string("hipGraphInstantiate: ") + hipGetErrorString(e));
    }
    *graph = new ftm_graph_s{g, x};
    g_last_error.clear();
    return FTM_OK;
}

int ftm_graph_launch(ftm_graph graph, hipStream_t stream) {
    if (!graph) return fail(FTM_ERR_INVALID_ARG, "ftm_graph_launch: graph is NULL");
    hipError_t e = hipGraphLaunch(graph->exec, (hipStream_t)stream);
    if (e != hipSuccess) return fail(FTM_ERR_HIP, std::string("hipGraphLaunch: ") + hipGetErrorString(e));
    g_last_error.clear();
    return FTM_OK;
}

int ftm_graph_destroy(ftm_graph graph) {
    if (!graph) return FTM_OK;
    hipError_t e1 = hipGraphExecDestroy(graph->exec);
    hipError_t e2 = hipGraphDestroy(graph->graph);
    delete graph;
    if (e1 != hipSuccess || e2 != hipSuccess)
        return fail(FTM_ERR_HIP, std::string("graph destroy: ") + hipGetErrorString(e1 != hipSuccess ? e1 : e2));
    return FTM_OK;
}

}  // extern "C"
