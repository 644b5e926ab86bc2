// C-ABI of the polymerized GEMM library: argument checks, plan cache,
// split-K workspaces, region launches and the offline calibration.
//
// Flow per call (MikPoly page, section 3 "complete algorithm" and section 4
// GPU platform): the shape becomes known -> the cached strategy for it is
// looked up, or built by the cost-model search on a miss -> every region's
// fixed-size micro-kernel is launched with the region's start addresses and
// trip counts as scalars; the hardware scheduler deals workgroups to CUs.
#include <dlfcn.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <array>
#include <atomic>
#include <chrono>
#include <climits>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <deque>
#include <fstream>
#include <functional>
#include <map>
#include <memory>
#include <mutex>
#include <shared_mutex>
#include <sstream>
#include <string>
#include <tuple>
#include <unordered_map>
#include <vector>

#include "../../include/mkp.h"
#include "kernels.h"
#include "planner.h"

namespace mkp {
namespace {

thread_local std::string t_last_error;
thread_local int64_t t_call = 0;   // sequence number of this thread's current GEMM call

int fail(int code, const std::string& msg) {
    t_last_error = msg;
    return code;
}

struct Key {
    int64_t batch, M, N, K;
    int align, device;
    bool bt;   // B given as N x K
    bool conv = false;   // implicit-GEMM convolution: single-tile plans, B as N x K, no transpose
    // > 0: at most this many K splits and no staging copies (a plan made to
    // fit the allocation-free entry point's fixed scratch)
    int cap = 0;
    bool operator==(const Key& o) const {
        return batch == o.batch && M == o.M && N == o.N && K == o.K && align == o.align && device == o.device &&
               bt == o.bt && conv == o.conv && cap == o.cap;
    }
};
struct KeyHash {
    size_t operator()(const Key& k) const {
        uint64_t h = 1469598103934665603ull;
        auto mix = [&](uint64_t v) {
            h ^= v;
            h *= 1099511628211ull;
        };
        mix((uint64_t)k.batch);
        mix((uint64_t)k.M);
        mix((uint64_t)k.N);
        mix((uint64_t)k.K);
        mix((uint64_t)k.align);
        mix((uint64_t)k.device);
        mix((uint64_t)k.bt);
        mix((uint64_t)k.conv);
        mix((uint64_t)k.cap);
        return (size_t)h;
    }
};

// One stream's scratch buffer.  `mu` is held by a call from the moment it
// takes the buffer until its last launch is enqueued, so calls that share a
// stream (from several threads) never interleave their use of it: one
// call's split-K partials cannot be overwritten, nor the buffer freed or
// regrown, between another call's launches.  Entries are never erased.
struct Workspace {
    std::mutex mu;
    void* ptr = nullptr;
    size_t bytes = 0;
};

// Split-K workspace layout: kCounterCap arrival counters (int32), then the
// partial tiles [splits][batch][m][ldw] (fp32, ldw = n rounded up to 4).
constexpr int kCounterCap = 1 << 16;
constexpr size_t kCounterBytes = (size_t)kCounterCap * 4;

struct TraceRec {
    int kernel;            // library kernel index, -1 = split-K reduction, -2 = zero fill, -3 = row pack
    int64_t call;          // sequence number of the C-ABI call that made the launch
    double flops, bytes;   // algorithmic work of the launch
    hipEvent_t e0, e1;
};

struct Library {
    std::shared_mutex mu;                         // guards table, opts, caches, generation
    // the active table: replaced whole (never modified), so a search can run
    // on a snapshot without holding `mu`
    std::shared_ptr<const PerfTable> table;
    int64_t generation = 0;                       // bumped whenever plans may change
    std::string table_origin = "analytic";
    SearchOptions opts;
    std::unordered_map<Key, std::shared_ptr<const Plan>, KeyHash> cache;
    std::deque<Key> cache_order;                  // insertion order: the oldest plan is evicted first
    std::map<std::vector<int64_t>, std::shared_ptr<const Plan>> gcache;   // grouped calls
    std::deque<std::vector<int64_t>> gcache_order;
    size_t cache_cap = 1 << 16;

    std::mutex ws_mu;
    // per device: 256 zero bytes, the source of a convolution's padding
    std::map<int, void*> zero_pages;
    // per (device, stream, slot): slot 0 serves the GEMM launches, slot 1
    // a convolution's channel-padded copies, which outlive slot 0's use
    // (a call that holds both takes slot 1 first)
    std::map<std::tuple<int, void*, int>, Workspace> workspaces;

    std::atomic<int64_t> hits{0}, misses{0}, launches{0};
    std::atomic<int64_t> plan_ns{0};

    // split-K: 0 = a second pass sums the partials; 1 = the last split of a
    // tile sums them after agent-scope fences
    std::atomic<int> fused_reduce{0};
    // store policy, bits: streaming stores for 1 final C whose rows are
    // whole 128-byte lines, 2 final C wherever 16-byte aligned, 4 split-K
    // partials; 8 only in regions of more than one wave, 16 only for a
    // region's C of at most 32 MB (the L2s' capacity); 32 split-K partials
    // written through to the level every XCD shares; 33 measured best
    std::atomic<int> nt_stores{33};
    std::atomic<bool> pack_unaligned{true};       // stage unaligned re-read operands aligned
    std::atomic<int> transpose_b{1};              // K x N calls as transpose + N x K: 0 no, 1 by cost, 2 always
    std::atomic<bool> trace{false};               // time every launch with events
    std::atomic<int64_t> calls{0};                // C-ABI GEMM calls so far
    std::mutex trace_mu;
    std::vector<TraceRec> trace_recs;
};

Library& lib() {
    static Library* L = new Library();  // never destroyed: safe at process exit
    return *L;
}

// ---- tables -----------------------------------------------------------------

// Analytic stand-in used until a measured table is loaded: MFMA time at a
// tile-size dependent efficiency vs. operand traffic, per K step.
PerfTable analytic_table() {
    PerfTable t;
    t.cus = 256;
    t.launch_us = 2.0;
    t.red_launch_us = 2.0;
    t.red_gbps = 4000.0;
    t.splits = {1, 2, 3, 4, 5, 6, 8, 12, 16, 24, 32};
    for (int i = 0; i < kernel_count(); ++i) {
        const KernelInfo& ki = kernel_info(i);
        TableKernel k;
        k.name = ki.name;
        k.uM = ki.uM;
        k.uN = ki.uN;
        k.uK = ki.uK;
        k.lib_index = i;
        k.bt = ki.bt;
        int by_lds = std::max(1, (160 * 1024) / std::max(ki.lds_bytes, 1));
        k.wg_per_cu = std::min(by_lds, 2);
        const double slots = (double)t.cus * k.wg_per_cu;
        const double area = (double)ki.uM * ki.uN;
        const double eff = 0.7 * std::min(1.0, std::pow(area / (256.0 * 256.0), 0.25));
        const double cu_rate = 4096.0 * 2400.0 * eff;                   // FLOP per us per CU
        const double t_c = k.wg_per_cu * 2.0 * ki.uM * ki.uN * ki.uK / cu_rate;
        const double t_m = slots * 2.0 * (ki.uM + ki.uN) * ki.uK / 12.0e6;  // ~12 TB/s via L2
        const double step = std::max(t_c, t_m);
        const double epi = slots * 4.0 * ki.uM * ki.uN / 6.0e6 + 0.5;
        for (int tt : {1, 2, 4, 8, 16, 32, 64, 128, 256}) k.pts.emplace_back((double)tt, epi + tt * step);
        t.kernels.push_back(k);
    }
    return t;
}

// Resolve table kernel names to library kernels.
// Library index of the two-tile kernel running kernels a then b (library
// indices) in one launch, or -1.
int dual_find(int a, int b) {
    if (a < 0 || b < 0) return -1;
    for (int i = 0; i < dual_count(); ++i) {
        const DualInfo& d = dual_info(i);
        if (kernel_find(d.first) == a && kernel_find(d.second) == b) return i;
    }
    return -1;
}

int conv_for(int lib);

bool bind_table(PerfTable& t, std::string& err) {
    for (auto& k : t.kernels) {
        k.lib_index = kernel_find(k.name.c_str());
        if (k.lib_index < 0) {
            err = "table names kernel '" + k.name + "' that the library does not have";
            return false;
        }
        const KernelInfo& ki = kernel_info(k.lib_index);
        if (ki.uM != k.uM || ki.uN != k.uN || ki.uK != k.uK || ki.bt != k.bt) {
            err = "table tile or layout of kernel '" + k.name + "' differs from the library's";
            return false;
        }
        k.conv_ok = conv_for(k.lib_index) >= 0;
    }
    // library kernels the table does not price (it was written before the
    // library had them) get the analytic estimates
    for (auto& k : analytic_table().kernels) {
        bool listed = false;
        for (auto& e : t.kernels) listed |= e.name == k.name;
        if (!listed) {
            t.kernels.push_back(k);
            t.kernels.back().conv_ok = conv_for(k.lib_index) >= 0;
        }
    }
    // kernel pairs: each listed pair must have a two-tile kernel; a table
    // without pair lines gets every pair the library has whose kernels it
    // prices with the same workgroups per CU
    for (auto& pr : t.pairs)
        if (dual_find(t.kernels[pr.first].lib_index, t.kernels[pr.second].lib_index) < 0) {
            err = "table pairs " + t.kernels[pr.first].name + " and " + t.kernels[pr.second].name +
                  ", which the library cannot run in one launch";
            return false;
        }
    if (t.pairs.empty())
        for (int d = 0; d < dual_count(); ++d) {
            int ia = -1, ib = -1;
            for (size_t i = 0; i < t.kernels.size(); ++i) {
                if (t.kernels[i].name == dual_info(d).first) ia = (int)i;
                if (t.kernels[i].name == dual_info(d).second) ib = (int)i;
            }
            if (ia >= 0 && ib >= 0 && t.kernels[ia].wg_per_cu == t.kernels[ib].wg_per_cu &&
                t.kernels[ia].bt == t.kernels[ib].bt)
                t.pairs.emplace_back(ia, ib);
        }
    return true;
}

// The analytic estimates with the library's kernel pairs bound.
PerfTable bound_analytic_table() {
    PerfTable t = analytic_table();
    std::string err;
    (void)bind_table(t, err);
    return t;
}

std::string default_table_path() {
    if (const char* e = std::getenv("MKP_CALIB")) return e;
    Dl_info info;
    if (dladdr((void*)&default_table_path, &info) && info.dli_fname) {
        std::string so = info.dli_fname;
        auto slash = so.rfind('/');
        std::string dir = slash == std::string::npos ? "." : so.substr(0, slash);
        return dir + "/calib/gfx950.tbl";
    }
    return "calib/gfx950.tbl";
}

bool read_file(const std::string& path, std::string& out) {
    std::ifstream f(path);
    if (!f) return false;
    std::stringstream ss;
    ss << f.rdbuf();
    out = ss.str();
    return true;
}

// Forget every cached plan (caller holds the lock exclusively); plans being
// built on an older snapshot are then not cached.
void clear_plans_locked(Library& L) {
    L.cache.clear();
    L.cache_order.clear();
    L.gcache.clear();
    L.gcache_order.clear();
    ++L.generation;
}

// Load the table at `path` (or the shipped one) into the library; caller holds the lock.
int load_table_locked(Library& L, const char* path, bool quiet_missing) {
    std::string p = path ? std::string(path) : default_table_path();
    std::string text, err;
    if (!read_file(p, text)) {
        // only a missing shipped table is quiet; a path the caller or
        // MKP_CALIB names must exist
        if (quiet_missing && !std::getenv("MKP_CALIB")) {
            L.table = std::make_shared<const PerfTable>(bound_analytic_table());
            L.table_origin = "analytic";
            clear_plans_locked(L);
            return MKP_OK;
        }
        return fail(MKP_ERR_INVALID_ARG, "cannot read performance table " + p);
    }
    PerfTable t;
    if (!parse_table(text, t, err) || !bind_table(t, err))
        return fail(MKP_ERR_INVALID_ARG, "performance table " + p + ": " + err);
    L.table = std::make_shared<const PerfTable>(std::move(t));
    L.table_origin = p;
    clear_plans_locked(L);
    return MKP_OK;
}

void read_env_options(Library& L) {
    if (const char* e = std::getenv("MKP_PATTERNS")) L.opts.allow_II = std::strstr(e, "II") != nullptr;
    if (const char* e = std::getenv("MKP_SPLITK_MAX")) L.opts.splitk_max = std::max(1, std::atoi(e));
    if (const char* e = std::getenv("MKP_FORCE_SPLITK")) L.opts.force_splitk = std::max(0, std::atoi(e));
    if (const char* e = std::getenv("MKP_CACHE_CAP")) L.cache_cap = (size_t)std::max(1, std::atoi(e));
    if (const char* e = std::getenv("MKP_NT_STORES")) L.nt_stores.store(std::min(63, std::max(0, std::atoi(e))));
    if (const char* e = std::getenv("MKP_FORCE_KERNEL")) {
        for (size_t i = 0; i < L.table->kernels.size(); ++i)
            if (L.table->kernels[i].name == e) L.opts.force_kernel = (int)i;
    }
}

std::once_flag g_init;
void ensure_init() {
    std::call_once(g_init, [] {
        Library& L = lib();
        std::unique_lock<std::shared_mutex> lk(L.mu);
        if (load_table_locked(L, nullptr, true) != MKP_OK) {
            // a shipped table that does not fit the library is a build error:
            // say so once, and plan with the analytic estimates
            std::fprintf(stderr, "libmkp: %s; planning with analytic estimates\n", t_last_error.c_str());
            L.table = std::make_shared<const PerfTable>(bound_analytic_table());
            L.table_origin = "analytic";
        }
        read_env_options(L);
    });
}

// ---- plans ------------------------------------------------------------------

// A snapshot of what a search needs, taken under the shared lock.
struct PlanInputs {
    std::shared_ptr<const PerfTable> table;
    SearchOptions opts;
    int transpose_mode = 0;
    int64_t generation = 0;
};

// Look the key up; on a miss, search on a snapshot with no lock held (so
// lookups of other shapes never wait behind a search) and cache the plan
// unless the table or the options changed meanwhile.
std::shared_ptr<const Plan> get_plan(const Key& key) {
    Library& L = lib();
    PlanInputs in;
    {
        std::shared_lock<std::shared_mutex> lk(L.mu);
        auto it = L.cache.find(key);
        if (it != L.cache.end()) {
            L.hits.fetch_add(1, std::memory_order_relaxed);
            return it->second;
        }
        in.table = L.table;
        in.opts = L.opts;
        in.generation = L.generation;
    }
    in.opts.bt = key.bt;
    in.opts.conv = key.conv;
    if (key.conv) in.opts.fuse = false;   // no two-tile form of the convolution kernels
    in.transpose_mode = key.conv ? 0 : key.batch <= 65535 ? L.transpose_b.load(std::memory_order_relaxed) : 0;
    if (key.cap > 0) {
        in.opts.splitk_max = std::min(in.opts.splitk_max, key.cap);
        in.opts.force_splitk = 0;
        in.transpose_mode = 0;
    }
    auto plan = std::make_shared<const Plan>(
        plan_call(*in.table, key.batch, key.M, key.N, key.K, in.opts, in.transpose_mode));
    L.misses.fetch_add(1, std::memory_order_relaxed);
    L.plan_ns.fetch_add((int64_t)(plan->plan_us * 1000.0), std::memory_order_relaxed);
    std::unique_lock<std::shared_mutex> lk(L.mu);
    if (L.generation != in.generation) return plan;
    auto ins = L.cache.emplace(key, plan);
    if (!ins.second) return ins.first->second;   // another thread cached it first
    L.cache_order.push_back(key);
    while (L.cache.size() > L.cache_cap && !L.cache_order.empty()) {
        L.cache.erase(L.cache_order.front());
        L.cache_order.pop_front();
    }
    return plan;
}

// ---- workspaces -------------------------------------------------------------

// A call's hold on one stream's workspace: from acquire() until the lease
// goes out of scope (after the call's last launch is enqueued), no other
// call takes the same (device, stream, slot) buffer.
class WsLease {
   public:
    WsLease() = default;
    WsLease(const WsLease&) = delete;
    WsLease& operator=(const WsLease&) = delete;

    // The buffer, at least `bytes` long (grown stream-ordered when short).
    int acquire(int dev, hipStream_t st, size_t bytes, void** out, int slot = 0) {
        Library& L = lib();
        if (!w_) {
            std::lock_guard<std::mutex> lk(L.ws_mu);
            w_ = &L.workspaces[{dev, (void*)st, slot}];
        }
        if (!lk_.owns_lock()) lk_ = std::unique_lock<std::mutex>(w_->mu);
        Workspace& w = *w_;
        if (w.bytes < bytes) {
            size_t want = std::max(bytes, w.bytes * 2);
            want = (want + 4095) & ~(size_t)4095;
            if (w.ptr) {
                hipError_t e = hipFreeAsync(w.ptr, st);
                w.ptr = nullptr;
                w.bytes = 0;
                if (e != hipSuccess) return fail(MKP_ERR_HIP, std::string("hipFreeAsync: ") + hipGetErrorString(e));
            }
            void* p = nullptr;
            hipError_t e = hipMallocAsync(&p, want, st);
            if (e != hipSuccess || !p) {
                (void)hipGetLastError();
                return fail(MKP_ERR_OOM, "split-K workspace of " + std::to_string(want) + " bytes: allocation failed");
            }
            // the fused reduction's arrival counters start at zero (and every
            // launch leaves them at zero)
            e = launch_zero_fill((float*)p, kCounterCap, 0, 1, kCounterCap, 1, st);
            if (e != hipSuccess) {
                (void)hipFreeAsync(p, st);
                return fail(MKP_ERR_HIP, std::string("workspace clear: ") + hipGetErrorString(e));
            }
            w.ptr = p;
            w.bytes = want;
        }
        *out = w.ptr;
        return MKP_OK;
    }

   private:
    Workspace* w_ = nullptr;
    std::unique_lock<std::mutex> lk_;
};

// Free every workspace (each after the calls holding it have enqueued their
// launches, and after the device has finished them).
void free_workspaces() {
    Library& L = lib();
    std::vector<std::pair<int, Workspace*>> all;
    {
        std::lock_guard<std::mutex> lk(L.ws_mu);
        for (auto& kv : L.workspaces) all.emplace_back(std::get<0>(kv.first), &kv.second);
    }
    if (all.empty()) return;
    int cur = 0;
    (void)hipGetDevice(&cur);
    for (auto& e : all) {
        std::lock_guard<std::mutex> lk(e.second->mu);
        if (!e.second->ptr) continue;
        (void)hipSetDevice(e.first);
        (void)hipDeviceSynchronize();
        (void)hipFree(e.second->ptr);
        e.second->ptr = nullptr;
        e.second->bytes = 0;
    }
    (void)hipSetDevice(cur);
}

// ---- dispatch ---------------------------------------------------------------

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Run one launch; in trace mode bracket it with events on the same stream.
template <class F>
hipError_t traced(Library& L, hipStream_t st, int kernel, double flops, double bytes, F&& fn) {
    if (!L.trace.load(std::memory_order_relaxed)) return fn();
    TraceRec r{kernel, t_call, flops, bytes, nullptr, nullptr};
    if (hipEventCreate(&r.e0) != hipSuccess || hipEventCreate(&r.e1) != hipSuccess) {
        if (r.e0) (void)hipEventDestroy(r.e0);
        return fn();
    }
    // the launch stamps the kernel's own start and end into the events
    // (the time between two events recorded on the stream around it would
    // also hold the dispatch gap before the kernel starts)
    launch_events() = LaunchEvents{r.e0, r.e1};
    hipError_t e = fn();
    const bool launched = launch_events().start == nullptr;
    launch_events() = LaunchEvents{};
    if (!launched || e != hipSuccess) {   // nothing was launched: no record
        (void)hipEventDestroy(r.e0);
        (void)hipEventDestroy(r.e1);
        return e;
    }
    std::lock_guard<std::mutex> lk(L.trace_mu);
    L.trace_recs.push_back(r);
    return e;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// C = A . B with B given as K x N (bt false) or as N x K (bt true, C = A . B^T
// of the stored matrix).
// Index of the convolution form of N x K kernel `lib`, or -1.
int conv_for(int lib) {
    if (lib < 0 || lib >= kernel_count()) return -1;
    for (int i = 0; i < conv_count(); ++i)
        if (std::strcmp(conv_info(i).twin, kernel_info(lib).name) == 0) return i;
    return -1;
}

// With `epi` (non-null) every final value goes through the fused epilogue.
// With `conv` (non-null) A is the NHWC input of an implicit-GEMM
// convolution (bt must be set: B is the KRSC filter bank).
// With `noalloc` the call's scratch is the library's fixed device array
// (kStaticScratchBytes): no allocation, and a plan whose scratch would not
// fit is replaced by one with fewer K splits and no staging copies.
int run_gemm(int64_t batch, int64_t M, int64_t N, int64_t K, const void* Av, int64_t lda, int64_t sA,
             const void* Bv, int64_t ldb, int64_t sB, float* C, int64_t ldc, int64_t sC, void* stream_v,
             bool bt = false, const KEpi* epi = nullptr, const KConv* conv = nullptr, bool noalloc = false) {
    if (batch < 0 || M < 0 || N < 0 || K < 0) return fail(MKP_ERR_INVALID_ARG, "negative dimension");
    if (M > INT_MAX || N > INT_MAX || K > INT_MAX) return fail(MKP_ERR_INVALID_ARG, "dimension exceeds 2^31-1");
    if (batch == 0 || M == 0 || N == 0) return MKP_OK;
    if (K > 0 && lda < K) return fail(MKP_ERR_INVALID_ARG, "lda < K");
    if (K > 0 && !bt && ldb < N) return fail(MKP_ERR_INVALID_ARG, "ldb < N");
    if (K > 0 && bt && ldb < K) return fail(MKP_ERR_INVALID_ARG, "ldb < K");
    if (ldc < N) return fail(MKP_ERR_INVALID_ARG, "ldc < N");
    if (!C) return fail(MKP_ERR_INVALID_ARG, "C is NULL");
    if (K > 0 && (!Av || !Bv)) return fail(MKP_ERR_INVALID_ARG, "A or B is NULL");
    if (batch > 1 && (sA < 0 || sB < 0 || sC < 0)) return fail(MKP_ERR_INVALID_ARG, "negative batch stride");
    ensure_init();
    t_call = lib().calls.fetch_add(1, std::memory_order_relaxed);
    hipStream_t st = (hipStream_t)stream_v;
    int dev = 0;
    hipError_t he = hipGetDevice(&dev);
    if (he != hipSuccess) return fail(MKP_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(he));

    Library& L = lib();
    // bytes the epilogue adds: the old C (beta != 0) and the bias vector
    const double epi_bytes =
        epi ? (epi->beta != 0.0f ? 4.0 * M * N * batch : 0.0) + (epi->bias ? 4.0 * N : 0.0) : 0.0;
    if (K == 0) {
        if (epi) {
            // empty sum: C := act(beta * C + bias)
            const bool vC0 = aligned16(C) && ldc % 4 == 0 && (batch == 1 || sC % 4 == 0);
            he = traced(L, st, -2, 0.0, 4.0 * M * N * batch + epi_bytes, [&] {
                return launch_splitk_reduce(nullptr, 0, 0, 0, 0, C, ldc, sC, (int)M, (int)N, (int)batch,
                                            vC0 ? 1 : 0, st, epi);
            });
        } else {
            he = traced(L, st, -2, 0.0, 4.0 * M * N * batch,
                        [&] { return launch_zero_fill(C, ldc, sC, (int)M, (int)N, (int)batch, st); });
        }
        if (he != hipSuccess) return fail(MKP_ERR_HIP, std::string("zero fill launch: ") + hipGetErrorString(he));
        L.launches.fetch_add(1, std::memory_order_relaxed);
        return MKP_OK;
    }
    if (batch > INT_MAX) return fail(MKP_ERR_INVALID_ARG, "batch exceeds 2^31-1");

    const uint16_t* A = (const uint16_t*)Av;
    const uint16_t* B = (const uint16_t*)Bv;
    // 128-bit loads need 16-byte aligned rows; the direct-load path also
    // keeps per-tile offsets (<= 256 rows of A, <= 64 rows of a K x N B,
    // <= 256 rows of an N x K B) in 32 bits
    // (convolution: 16-byte aligned input with C % 8 == 0, so 8 channels of
    // one tap are 16 aligned bytes)
    bool vA = conv ? aligned16(A) && conv->C % 8 == 0
                   : aligned16(A) && lda % 8 == 0 && (batch == 1 || sA % 8 == 0) && lda < (int64_t(1) << 23);
    bool vB = aligned16(B) && ldb % 8 == 0 && (batch == 1 || sB % 8 == 0) &&
              ldb < (int64_t(1) << (bt ? 23 : 25));
    const bool vC = aligned16(C) && ldc % 4 == 0 && (batch == 1 || sC % 4 == 0);
    const int align = (vA ? 1 : 0) | (vB ? 2 : 0) | (vC ? 4 : 0);

    Key key{batch, M, N, K, align, dev, bt, conv != nullptr};
    std::shared_ptr<const Plan> plan = get_plan(key);
    if (plan->regions.empty()) {
        if (plan->rank > 0)
            return fail(MKP_ERR_UNSUPPORTED, "plan_rank " + std::to_string(plan->rank) + " beyond the " +
                                                 std::to_string(plan->candidates) + " candidates of this shape");
        return fail(MKP_ERR_UNSUPPORTED, "no plan for this shape");
    }

    // An operand with unaligned rows that several tile rows (columns) re-read
    // is first copied into a staging buffer with rows padded to 8 elements
    // (as the Bolt page pads kernels to alignment 8), so the micro-kernels
    // take the direct-load path.  Workspace layout, regions in order on one
    // stream sharing it: [split-K counters][split-K partials][A copy][B copy].
    // The two regions of a one-launch plan run together: each gets its own
    // partial area and its own range of counters.
    // A K x N B the plan runs on N x K kernels is first transposed into the
    // workspace (rows of K padded to 8 elements, aligned)
    const int64_t ldt = (K + 7) & ~int64_t(7);
    // B rows: N long for a K x N B, K long for an N x K one
    const int64_t b_rows = bt ? N : K, b_cols = bt ? K : N;
    const int64_t ldap = (K + 7) & ~int64_t(7), ldbp = (b_cols + 7) & ~int64_t(7);
    // (a copy pays off once several tile rows/columns re-read the operand
    // and K is deep enough that the element loads it saves outweigh its
    // launch: measured, batched 505 x 505 x 64 calls run 7 % faster without
    // the copy and 8 x (777 x 777 x 777) 26 % faster with it)
    constexpr int64_t kPackMinK = 512;
    auto round256 = [](size_t x) { return (x + 255) & ~size_t(255); };
    struct Layout {
        bool one_launch = false, tr = false, packA = false, packB = false;
        size_t part_bytes = 0, part_off[2] = {0, 0};
        size_t offA = 0, offB = 0, ws_bytes = 0;
    };
    auto layout_of = [&](const Plan& p, bool copies_ok) {
        Layout w;
        w.one_launch = !conv && p.fused && p.regions.size() == 2;
        for (size_t i = 0; i < p.regions.size() && i < 2; ++i) {
            const Region& r = p.regions[i];
            if (r.s <= 1) continue;
            const int64_t ldw = (r.n + 3) & ~int64_t(3);
            const size_t bytes = (size_t)r.s * (size_t)batch * (size_t)r.m * (size_t)ldw * sizeof(float);
            if (w.one_launch) {
                w.part_off[i] = i == 0 ? 0 : round256(w.part_bytes);
                w.part_bytes = w.part_off[i] + bytes;
            } else {
                w.part_bytes = std::max(w.part_bytes, bytes);
            }
        }
        const bool pack_on = copies_ok && L.pack_unaligned.load(std::memory_order_relaxed);
        w.tr = p.transpose_b && !bt;
        w.packA = !conv && pack_on && !vA && N > 192 && K >= kPackMinK && ldap < (int64_t(1) << 23);
        w.packB = !w.tr && pack_on && !vB && M > 192 && K >= kPackMinK && ldbp < (int64_t(1) << (bt ? 23 : 25));
        w.offA = kCounterBytes + round256(w.part_bytes);
        const size_t bytesA = w.packA ? (size_t)batch * M * ldap * 2 : 0;
        w.offB = w.offA + round256(bytesA);
        const size_t bytesB = w.tr ? (size_t)batch * N * ldt * 2 : w.packB ? (size_t)batch * b_rows * ldbp * 2 : 0;
        w.ws_bytes = (w.part_bytes || w.packA || w.packB || w.tr) ? w.offB + bytesB : 0;
        return w;
    };
    Layout lay = layout_of(*plan, true);
    if (noalloc && lay.ws_bytes > kStaticScratchBytes) {
        // fewer K splits and no copies, until the scratch fits
        int most = 1;
        for (const Region& r : plan->regions) most = std::max(most, r.s);
        for (int cap = std::max(1, most / 2);; cap = std::max(1, cap / 2)) {
            Key k2 = key;
            k2.cap = cap;
            plan = get_plan(k2);
            if (plan->regions.empty()) return fail(MKP_ERR_UNSUPPORTED, "no plan for this shape");
            lay = layout_of(*plan, false);
            if (lay.ws_bytes <= kStaticScratchBytes || cap == 1) break;
        }
        if (lay.ws_bytes > kStaticScratchBytes)
            return fail(MKP_ERR_UNSUPPORTED, "the call needs " + std::to_string(lay.ws_bytes) +
                                                 " bytes of scratch, more than the " +
                                                 std::to_string(kStaticScratchBytes) +
                                                 " bytes of the allocation-free entry point");
    }
    const bool one_launch = lay.one_launch, tr = lay.tr, packA = lay.packA, packB = lay.packB;
    const size_t part_off[2] = {lay.part_off[0], lay.part_off[1]};
    const size_t offA = lay.offA, offB = lay.offB, ws_bytes = lay.ws_bytes;
    void* ws = nullptr;
    WsLease lease;   // held until this call's last launch is enqueued
    if (ws_bytes && noalloc) {
        // the fixed array of this device (calls that overlap on one GPU share it)
        he = static_scratch(dev, &ws);
        if (he != hipSuccess)
            return fail(MKP_ERR_HIP, std::string("scratch address: ") + hipGetErrorString(he));
    } else if (ws_bytes) {
        int rc = lease.acquire(dev, st, ws_bytes, &ws);
        if (rc != MKP_OK) return rc;
    }
    if (packA) {
        uint16_t* dst = (uint16_t*)((char*)ws + offA);
        he = traced(L, st, -3, 0.0, (double)batch * M * (2.0 * K + 2.0 * ldap),
                    [&] { return launch_pack_rows(A, lda, sA, dst, ldap, (int)M, (int)K, (int)batch, st); });
        if (he != hipSuccess) return fail(MKP_ERR_HIP, std::string("pack launch: ") + hipGetErrorString(he));
        A = dst;
        lda = ldap;
        sA = M * ldap;
        vA = true;
    }
    if (tr) {
        uint16_t* dst = (uint16_t*)((char*)ws + offB);
        he = traced(L, st, -4, 0.0, (double)batch * (2.0 * K * N + 2.0 * N * ldt), [&] {
            return launch_transpose_bf16(B, ldb, sB, dst, ldt, N * ldt, (int)K, (int)N, (int)batch, vB, st);
        });
        if (he != hipSuccess) return fail(MKP_ERR_HIP, std::string("transpose launch: ") + hipGetErrorString(he));
        L.launches.fetch_add(1, std::memory_order_relaxed);
        B = dst;
        ldb = ldt;
        sB = N * ldt;
        vB = true;
    }
    const bool kbt = bt || tr;   // the regions' kernels take B as N x K
    if (packB) {
        uint16_t* dst = (uint16_t*)((char*)ws + offB);
        he = traced(L, st, -3, 0.0, (double)batch * b_rows * (2.0 * b_cols + 2.0 * ldbp), [&] {
            return launch_pack_rows(B, ldb, sB, dst, ldbp, (int)b_rows, (int)b_cols, (int)batch, st);
        });
        if (he != hipSuccess) return fail(MKP_ERR_HIP, std::string("pack launch: ") + hipGetErrorString(he));
        B = dst;
        ldb = ldbp;
        sB = b_rows * ldbp;
        vB = true;
    }

    // One region's launch arguments; `counter0`: its first split-K counter.
    struct RegionLaunch {
        KArgs a{};
        KEpi e{};
        const KernelInfo* ki = nullptr;
        bool fused_red = false;   // split-K reduced by the last-arriving split
        bool ntC = false;         // final C through streaming stores
        bool ntRed = false;       // ... also from the second pass
        float* Creg = nullptr;
        int64_t ldw = 0, G = 0;
        double flops = 0, bytes = 0, red_bytes = 0;
    };
    auto setup = [&](size_t i, int64_t counter0, int64_t counter_cap, RegionLaunch& R) -> int {
        const Region& r = plan->regions[i];
        const int li = r.lib;
        if (li < 0 || li >= kernel_count()) return fail(MKP_ERR_UNSUPPORTED, "plan kernel is not launchable");
        const KernelInfo& ki = kernel_info(li);
        if (ki.bt != kbt) return fail(MKP_ERR_UNSUPPORTED, "plan kernel has the other B layout");
        R.ki = &ki;
        KArgs& a = R.a;
        a.A = conv ? A : A + r.m0 * lda;
        if (conv) {
            a.conv = *conv;
            a.conv.m0 = (int)r.m0;
        }
        a.B = kbt ? B + r.n0 * ldb : B + r.n0;
        a.lda = lda;
        a.ldb = ldb;
        a.sA = sA;
        a.sB = sB;
        a.M = (int)r.m;
        a.N = (int)r.n;
        a.K = (int)K;
        a.tiles_m = (int)ceil_div(r.m, ki.uM);
        a.tiles_n = (int)ceil_div(r.n, ki.uN);
        a.steps_per_split = r.steps;
        a.splits = r.s;
        a.batch = (int)batch;
        a.flags = (vA ? KF_VEC_A : 0) | (vB ? KF_VEC_B : 0);
        // (the direct-load gather keeps input offsets in 32 bits: from tap
        // (0, 0) of the first pixel, up to pad rows/columns before the
        // image, to the last tap of the last one)
        if (conv && vA && conv->C % ki.uK == 0) {
            const int64_t imgs = M / ((int64_t)conv->P * conv->Q);
            const int64_t span = imgs * ((int64_t)conv->H + 2 * conv->ph + (int64_t)conv->dh * conv->R) *
                                 ((int64_t)conv->W + 2 * conv->pw + (int64_t)conv->dw * conv->S) * conv->C;
            if (span < INT_MAX / 2) a.flags |= KF_CONV_DMA;
        }
        R.Creg = C + r.m0 * ldc + r.n0;
        R.ldw = (r.n + 3) & ~int64_t(3);
        // streaming stores for the region's final C and for its split-K
        // partials, as the option's bits select
        // (the streaming stores take 32-bit byte offsets from a tile's
        // origin, or from C's for the second pass)
        const int nt_mode = L.nt_stores.load(std::memory_order_relaxed);
        const bool nt_here = (!(nt_mode & 8) || r.waves > 1) &&
                             (!(nt_mode & 16) || 4.0 * r.m * r.n * batch <= 32.0 * 1024 * 1024);
        R.ntC = nt_here && vC && ldc * 256 * 4 < (int64_t(1) << 31) &&
                ((nt_mode & 2) || ((nt_mode & 1) && ldc % 32 == 0 && (batch == 1 || sC % 32 == 0) &&
                                   ((uintptr_t)R.Creg & 127) == 0));
        R.ntRed = R.ntC && ((batch - 1) * sC + r.m * ldc) * 4 < (int64_t(1) << 31);
        if (r.s == 1) {
            a.C = R.Creg;
            a.ldc = ldc;
            a.sC = sC;
            a.sCsplit = 0;
            a.flags |= vC ? KF_VEC_C : 0;
            a.flags |= R.ntC ? KF_NT_C : 0;
        } else {
            a.C = (float*)((char*)ws + kCounterBytes + part_off[i < 2 ? i : 0]);
            a.ldc = R.ldw;
            a.sC = r.m * R.ldw;
            a.sCsplit = batch * r.m * R.ldw;
            a.flags |= KF_VEC_C;
            a.flags |= (nt_here && (nt_mode & 4) && R.ldw * 256 * 4 < (int64_t(1) << 31)) ? KF_NT_C : 0;
            a.flags |= (nt_here && (nt_mode & 32) && R.ldw * 256 * 4 < (int64_t(1) << 31)) ? KF_SC1_C : 0;
        }
        // fused reduction when the per-tile counters fit, else a second pass
        const int64_t ntiles = (int64_t)a.tiles_m * a.tiles_n * batch;
        // (the allocation-free call sums splits in a second pass: its
        // scratch then holds nothing that must start at zero)
        // (its partial stores and loads take 32-bit byte offsets within a
        // tile: 256 rows of ldw floats)
        R.fused_red = r.s > 1 && ki.fused_ok && !noalloc && L.fused_reduce.load(std::memory_order_relaxed) == 1 &&
                      counter0 + ntiles <= counter_cap && R.ldw * 256 * 4 < (int64_t(1) << 31);
        a.counters = R.fused_red ? (int*)ws + counter0 : nullptr;
        a.Cout = R.Creg;
        a.ldcout = ldc;
        a.sCout = sC;
        if (vC) a.flags |= KF_VEC_COUT;
        // the epilogue's bias starts at the region's first column; it runs in
        // the micro-kernel unless a second pass reduces the splits
        if (epi) {
            R.e = *epi;
            if (R.e.bias) R.e.bias += r.n0;
            if (r.s == 1 || R.fused_red) {
                a.flags |= KF_EPI;
                a.epi = R.e;
            }
        }
        const double r_epi = epi ? (epi->beta != 0.0f ? 4.0 * r.m * r.n * batch : 0.0) + (epi->bias ? 4.0 * r.n : 0.0)
                                 : 0.0;
        R.G = (int64_t)a.tiles_m * a.tiles_n * a.splits * batch;
        if (R.G > INT_MAX) return fail(MKP_ERR_UNSUPPORTED, "grid too large");
        R.flops = 2.0 * r.m * r.n * K * batch;
        R.bytes = (double)batch * (2.0 * r.m * K + 2.0 * K * r.n + 4.0 * r.m * r.n) + ((a.flags & KF_EPI) ? r_epi : 0.0);
        if (conv)   // the region's share of the input, its filters and its output, once each
            R.bytes = 2.0 * (double)(M / ((int64_t)conv->P * conv->Q)) * conv->H * conv->W * conv->C * r.m / M +
                      2.0 * K * r.n + 4.0 * r.m * r.n + ((a.flags & KF_EPI) ? r_epi : 0.0);
        R.red_bytes = (double)(r.s + 1) * 4.0 * r.m * r.n * batch + (epi ? r_epi : 0.0);
        return MKP_OK;
    };
    auto reduce = [&](size_t i, RegionLaunch& R) -> int {
        const Region& r = plan->regions[i];
        if (r.s <= 1 || R.fused_red) return MKP_OK;
        he = traced(L, st, -1, 0.0, R.red_bytes, [&] {
            return launch_splitk_reduce(R.a.C, r.s, batch * r.m * R.ldw, r.m * R.ldw, R.ldw, R.Creg, ldc, sC, (int)r.m,
                                        (int)r.n, (int)batch, (vC ? 1 : 0) | (R.ntRed ? 2 : 0), st,
                                        epi ? &R.e : nullptr);
        });
        if (he != hipSuccess) return fail(MKP_ERR_HIP, std::string("reduce launch: ") + hipGetErrorString(he));
        L.launches.fetch_add(1, std::memory_order_relaxed);
        return MKP_OK;
    };

    if (one_launch) {
        // both regions in one launch of the pair's two-tile kernel
        RegionLaunch R[2];
        int rc = setup(0, 0, kCounterCap, R[0]);
        if (rc != MKP_OK) return rc;
        const int64_t used = R[0].fused_red ? (int64_t)R[0].a.tiles_m * R[0].a.tiles_n * batch : 0;
        rc = setup(1, used, kCounterCap, R[1]);
        if (rc != MKP_OK) return rc;
        const int d = dual_find(plan->regions[0].lib, plan->regions[1].lib);
        if (d < 0) return fail(MKP_ERR_UNSUPPORTED, "plan pairs kernels that have no one-launch form");
        const int64_t G = R[0].G + R[1].G;
        if (G > INT_MAX) return fail(MKP_ERR_UNSUPPORTED, "grid too large");
        he = traced(L, st, -100 - d, R[0].flops + R[1].flops, R[0].bytes + R[1].bytes, [&] {
            return dual_info(d).launch(R[0].a, R[1].a, (int)R[0].G, dim3((unsigned)G), st);
        });
        if (he != hipSuccess) return fail(MKP_ERR_HIP, std::string("kernel launch: ") + hipGetErrorString(he));
        L.launches.fetch_add(1, std::memory_order_relaxed);
        for (size_t i = 0; i < 2; ++i)
            if ((rc = reduce(i, R[i])) != MKP_OK) return rc;
        return MKP_OK;
    }
    for (size_t i = 0; i < plan->regions.size(); ++i) {
        RegionLaunch R;
        int rc = setup(i, 0, kCounterCap, R);
        if (rc != MKP_OK) return rc;
        auto launch = R.ki->launch;
        if (conv) {
            const int ci = conv_for(plan->regions[i].lib);
            if (ci < 0) return fail(MKP_ERR_UNSUPPORTED, "plan kernel has no convolution form");
            launch = conv_info(ci).launch;
        }
        he = traced(L, st, plan->regions[i].lib, R.flops, R.bytes,
                    [&] { return launch(R.a, dim3((unsigned)R.G), st); });
        if (he != hipSuccess) return fail(MKP_ERR_HIP, std::string("kernel launch: ") + hipGetErrorString(he));
        L.launches.fetch_add(1, std::memory_order_relaxed);
        if ((rc = reduce(i, R)) != MKP_OK) return rc;
    }
    return MKP_OK;
}

// C_g := A . B_g for g < G (shared A, K; B_g K x N_g, or N_g x K when bt).
int run_grouped(int64_t G, int64_t M, int64_t K, const void* Av, int64_t lda, const int64_t* Ns,
                const void* const* Bs, const int64_t* ldbs, float* const* Cs, const int64_t* ldcs, void* stream_v,
                bool bt) {
    if (G < 1 || G > kMaxGroups) return fail(MKP_ERR_INVALID_ARG, "groups must be 1.." + std::to_string(kMaxGroups));
    if (!Ns || !Bs || !ldbs || !Cs || !ldcs) return fail(MKP_ERR_INVALID_ARG, "group arrays are NULL");
    if (M < 0 || K < 0) return fail(MKP_ERR_INVALID_ARG, "negative dimension");
    if (M > INT_MAX || K > INT_MAX) return fail(MKP_ERR_INVALID_ARG, "dimension exceeds 2^31-1");
    for (int64_t g = 0; g < G; ++g) {
        const int64_t N = Ns[g];
        if (N < 0) return fail(MKP_ERR_INVALID_ARG, "negative dimension");
        if (N > INT_MAX) return fail(MKP_ERR_INVALID_ARG, "dimension exceeds 2^31-1");
        if (N == 0 || M == 0) continue;
        if (K > 0 && (bt ? ldbs[g] < K : ldbs[g] < N)) return fail(MKP_ERR_INVALID_ARG, bt ? "ldb < K" : "ldb < N");
        if (ldcs[g] < N) return fail(MKP_ERR_INVALID_ARG, "ldc < N");
        if (!Cs[g]) return fail(MKP_ERR_INVALID_ARG, "C is NULL");
        if (K > 0 && !Bs[g]) return fail(MKP_ERR_INVALID_ARG, "B is NULL");
    }
    if (K > 0 && M > 0 && lda < K) return fail(MKP_ERR_INVALID_ARG, "lda < K");
    if (K > 0 && M > 0 && !Av) return fail(MKP_ERR_INVALID_ARG, "A is NULL");
    // the groups that have work
    std::vector<int64_t> live;
    for (int64_t g = 0; g < G; ++g)
        if (Ns[g] > 0) live.push_back(g);
    if (M == 0 || live.empty()) return MKP_OK;
    ensure_init();
    t_call = lib().calls.fetch_add(1, std::memory_order_relaxed);
    hipStream_t st = (hipStream_t)stream_v;
    int dev = 0;
    hipError_t he = hipGetDevice(&dev);
    if (he != hipSuccess) return fail(MKP_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(he));
    Library& L = lib();
    if (K == 0) {
        for (int64_t g : live) {
            he = traced(L, st, -2, 0.0, 4.0 * M * Ns[g],
                        [&] { return launch_zero_fill(Cs[g], ldcs[g], 0, (int)M, (int)Ns[g], 1, st); });
            if (he != hipSuccess) return fail(MKP_ERR_HIP, std::string("zero fill launch: ") + hipGetErrorString(he));
            L.launches.fetch_add(1, std::memory_order_relaxed);
        }
        return MKP_OK;
    }
    // plan (cached by M, K, layout, device and the group widths)
    std::vector<int64_t> key{M, K, bt ? 1 : 0, dev};
    std::vector<int64_t> widths;
    for (int64_t g : live) {
        key.push_back(Ns[g]);
        widths.push_back(Ns[g]);
    }
    std::shared_ptr<const Plan> plan;
    PlanInputs in;
    {
        std::shared_lock<std::shared_mutex> lk(L.mu);
        auto it = L.gcache.find(key);
        if (it != L.gcache.end()) plan = it->second;
        in.table = L.table;
        in.opts = L.opts;
        in.generation = L.generation;
    }
    if (plan) {
        L.hits.fetch_add(1, std::memory_order_relaxed);
    } else {
        // searched with no lock held, cached unless the table or options changed
        in.opts.bt = bt;
        plan = std::make_shared<const Plan>(polymerize_grouped(*in.table, M, K, widths, in.opts));
        L.misses.fetch_add(1, std::memory_order_relaxed);
        L.plan_ns.fetch_add((int64_t)(plan->plan_us * 1000.0), std::memory_order_relaxed);
        std::unique_lock<std::shared_mutex> lk(L.mu);
        if (L.generation == in.generation) {
            auto ins = L.gcache.emplace(key, plan);
            if (!ins.second) {
                plan = ins.first->second;
            } else {
                L.gcache_order.push_back(key);
                while (L.gcache.size() > L.cache_cap && !L.gcache_order.empty()) {
                    L.gcache.erase(L.gcache_order.front());
                    L.gcache_order.pop_front();
                }
            }
        }
    }
    if (plan->regions.empty()) return fail(MKP_ERR_UNSUPPORTED, "no plan for this grouped call");
    const Region& r = plan->regions[0];
    if (r.lib < 0 || r.lib >= kernel_count()) return fail(MKP_ERR_UNSUPPORTED, "plan kernel is not launchable");
    const KernelInfo& ki = kernel_info(r.lib);
    if (ki.bt != bt) return fail(MKP_ERR_UNSUPPORTED, "plan kernel has the other B layout");

    const uint16_t* A = (const uint16_t*)Av;
    const bool vA = aligned16(A) && lda % 8 == 0 && lda < (int64_t(1) << 23);
    KArgs a{};
    a.A = A;
    a.lda = lda;
    a.M = (int)M;
    a.K = (int)K;
    a.tiles_m = (int)ceil_div(M, ki.uM);
    a.steps_per_split = r.steps;
    a.splits = r.s;
    a.batch = 1;
    a.flags = vA ? KF_VEC_A : 0;
    a.ngroups = (int)live.size();
    // the store policy of a plain call, applied per group (its C) and to the
    // shared split-K workspace
    const int nt_mode = L.nt_stores.load(std::memory_order_relaxed);
    int64_t cbytes = 0;
    for (int64_t g : live) cbytes += 4 * M * Ns[g];
    const bool nt_here = (!(nt_mode & 8) || r.waves > 1) && (!(nt_mode & 16) || cbytes <= 32 * 1024 * 1024);
    std::vector<bool> ntRed(live.size(), false);
    int tile0 = 0;
    double flops = 0, bytes = 2.0 * M * K;
    for (size_t i = 0; i < live.size(); ++i) {
        const int64_t g = live[i];
        KGroup& G_ = a.group[i];
        G_.B = (const uint16_t*)Bs[g];
        G_.C = Cs[g];
        G_.ldb = ldbs[g];
        G_.ldc = ldcs[g];
        G_.N = (int)Ns[g];
        G_.tile0 = tile0;
        const bool vB = aligned16(Bs[g]) && ldbs[g] % 8 == 0 && ldbs[g] < (int64_t(1) << (bt ? 23 : 25));
        const bool vC = aligned16(Cs[g]) && ldcs[g] % 4 == 0;
        // (streaming stores take 32-bit byte offsets from a tile's origin,
        // or from the group's C in the second pass)
        const bool ntC = nt_here && vC && ldcs[g] * 256 * 4 < (int64_t(1) << 31) &&
                         ((nt_mode & 2) || ((nt_mode & 1) && ldcs[g] % 32 == 0 && ((uintptr_t)Cs[g] & 127) == 0));
        ntRed[i] = ntC && M * ldcs[g] * 4 < (int64_t(1) << 31);
        G_.flags = (vB ? KF_VEC_B : 0) | (vC ? KF_VEC_C : 0) | (ntC ? KF_NT_C : 0);
        tile0 += (int)ceil_div(Ns[g], ki.uN);
        flops += 2.0 * M * Ns[g] * K;
        bytes += 2.0 * K * Ns[g] + 4.0 * M * Ns[g];
    }
    a.tiles_n = tile0;
    // split-K partials: one workspace whose columns follow the launch's tile columns
    const int64_t ldw = (int64_t)tile0 * ki.uN;
    float* W = nullptr;
    WsLease lease;   // held until this call's last launch is enqueued
    if (r.s > 1) {
        void* ws = nullptr;
        int rc = lease.acquire(dev, st, kCounterBytes + (size_t)r.s * M * ldw * sizeof(float), &ws);
        if (rc != MKP_OK) return rc;
        W = (float*)((char*)ws + kCounterBytes);
        a.C = W;
        a.ldc = ldw;
        a.sC = M * ldw;
        a.sCsplit = M * ldw;
        a.flags |= KF_VEC_C;
        a.flags |= (nt_here && (nt_mode & 4) && ldw * 256 * 4 < (int64_t(1) << 31)) ? KF_NT_C : 0;
        a.flags |= (nt_here && (nt_mode & 32) && ldw * 256 * 4 < (int64_t(1) << 31)) ? KF_SC1_C : 0;
    }
    const int64_t grid = (int64_t)a.tiles_m * a.tiles_n * a.splits;
    if (grid > INT_MAX) return fail(MKP_ERR_UNSUPPORTED, "grid too large");
    he = traced(L, st, r.lib, flops, bytes, [&] { return ki.launch(a, dim3((unsigned)grid), st); });
    if (he != hipSuccess) return fail(MKP_ERR_HIP, std::string("kernel launch: ") + hipGetErrorString(he));
    L.launches.fetch_add(1, std::memory_order_relaxed);
    if (r.s > 1) {
        for (size_t i = 0; i < live.size(); ++i) {
            const KGroup& G_ = a.group[i];
            he = traced(L, st, -1, 0.0, (double)(r.s + 1) * 4.0 * M * G_.N, [&] {
                return launch_splitk_reduce(W + (int64_t)G_.tile0 * ki.uN, r.s, M * ldw, 0, ldw, G_.C, G_.ldc, 0,
                                            (int)M, G_.N, 1, ((G_.flags & KF_VEC_C) ? 1 : 0) | (ntRed[i] ? 2 : 0), st);
            });
            if (he != hipSuccess) return fail(MKP_ERR_HIP, std::string("reduce launch: ") + hipGetErrorString(he));
            L.launches.fetch_add(1, std::memory_order_relaxed);
        }
    }
    return MKP_OK;
}

int write_out(const std::string& s, char* buf, size_t len) {
    if (!buf || len == 0) return fail(MKP_ERR_BUFFER, "output buffer is empty");
    if (s.size() + 1 > len) {
        std::memcpy(buf, s.data(), len - 1);
        buf[len - 1] = 0;
        return fail(MKP_ERR_BUFFER, "output buffer too small: need " + std::to_string(s.size() + 1));
    }
    std::memcpy(buf, s.c_str(), s.size() + 1);
    return MKP_OK;
}

// ---- calibration ------------------------------------------------------------

double time_launches(const std::function<hipError_t()>& fn, int warm, int reps, hipError_t* err) {
    *err = hipSuccess;
    for (int i = 0; i < warm; ++i)
        if ((*err = fn()) != hipSuccess) return 0;
    hipEvent_t e0, e1;
    (void)hipEventCreate(&e0);
    (void)hipEventCreate(&e1);
    (void)hipEventRecord(e0, nullptr);
    for (int i = 0; i < reps; ++i)
        if ((*err = fn()) != hipSuccess) break;
    (void)hipEventRecord(e1, nullptr);
    (void)hipEventSynchronize(e1);
    float ms = 0;
    (void)hipEventElapsedTime(&ms, e0, e1);
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    return 1000.0 * ms / reps;
}

}  // namespace
}  // namespace mkp

using namespace mkp;

extern "C" {

int mkp_gemm(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb, float* C,
             int64_t ldc, void* stream) {
    return run_gemm(1, M, N, K, A, lda, 0, B, ldb, 0, C, ldc, 0, stream);
}

int mkp_gemm_batched(int64_t batch, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, int64_t strideA,
                     const void* B, int64_t ldb, int64_t strideB, float* C, int64_t ldc, int64_t strideC,
                     void* stream) {
    return run_gemm(batch, M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc, strideC, stream);
}

int mkp_gemm_batched_noalloc(int64_t batch, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                             int64_t strideA, const void* B, int64_t ldb, int64_t strideB, float* C, int64_t ldc,
                             int64_t strideC, void* stream) {
    return run_gemm(batch, M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc, strideC, stream, false, nullptr, nullptr,
                    true);
}

size_t mkp_noalloc_scratch_bytes(void) { return kStaticScratchBytes; }

int mkp_gemm_bt(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb, float* C,
                int64_t ldc, void* stream) {
    return run_gemm(1, M, N, K, A, lda, 0, B, ldb, 0, C, ldc, 0, stream, true);
}

int mkp_gemm_batched_bt(int64_t batch, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                        int64_t strideA, const void* B, int64_t ldb, int64_t strideB, float* C, int64_t ldc,
                        int64_t strideC, void* stream) {
    return run_gemm(batch, M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc, strideC, stream, true);
}

// 256 zero bytes on device `dev` (allocated and cleared on first use).
int zero_page(int dev, const uint16_t** out) {
    Library& L = lib();
    std::lock_guard<std::mutex> lk(L.ws_mu);
    void*& p = L.zero_pages[dev];
    if (!p) {
        void* q = nullptr;
        hipError_t e = hipMalloc(&q, 256);
        if (e != hipSuccess || !q) {
            (void)hipGetLastError();
            return fail(MKP_ERR_OOM, "zero page: allocation failed");
        }
        e = hipMemset(q, 0, 256);
        if (e != hipSuccess) {
            (void)hipFree(q);
            return fail(MKP_ERR_HIP, std::string("zero page: ") + hipGetErrorString(e));
        }
        p = q;
    }
    *out = (const uint16_t*)p;
    return MKP_OK;
}

int mkp_conv2d(int64_t N, int64_t H, int64_t W, int64_t C, int64_t K, int64_t R, int64_t S, int64_t stride_h,
               int64_t stride_w, int64_t pad_h, int64_t pad_w, int64_t dil_h, int64_t dil_w, const void* x,
               const void* w, float* y, const float* bias, int act, void* stream) {
    if (N < 0 || K < 0 || H < 1 || W < 1 || C < 1 || R < 1 || S < 1)
        return fail(MKP_ERR_INVALID_ARG, "bad dimension (H, W, C, R, S >= 1; N, K >= 0)");
    if (stride_h < 1 || stride_w < 1 || dil_h < 1 || dil_w < 1 || pad_h < 0 || pad_w < 0)
        return fail(MKP_ERR_INVALID_ARG, "strides and dilations must be >= 1, padding >= 0");
    if (act < 0 || act >= ACT_COUNT) return fail(MKP_ERR_INVALID_ARG, "unknown activation");
    const int64_t span_h = dil_h * (R - 1) + 1, span_w = dil_w * (S - 1) + 1;
    if (H + 2 * pad_h < span_h || W + 2 * pad_w < span_w)
        return fail(MKP_ERR_INVALID_ARG, "filter larger than the padded input");
    const int64_t P = (H + 2 * pad_h - span_h) / stride_h + 1, Q = (W + 2 * pad_w - span_w) / stride_w + 1;
    if (N == 0 || K == 0) return MKP_OK;
    const int64_t M = N * P * Q, Kg = R * S * C;
    if (M > INT_MAX || Kg > INT_MAX || N * H > INT_MAX || H > INT_MAX / 4 || W > INT_MAX / 4 || C > INT_MAX / 4 ||
        pad_h > INT_MAX / 4 || pad_w > INT_MAX / 4 || stride_h * P > INT_MAX / 4 || stride_w * Q > INT_MAX / 4 ||
        dil_h * R > INT_MAX / 4 || dil_w * S > INT_MAX / 4)
        return fail(MKP_ERR_INVALID_ARG, "convolution extents exceed the 32-bit index range");
    if (!x || !w || !y) return fail(MKP_ERR_INVALID_ARG, "x, w or y is NULL");
    const KEpi e{bias, 1.0f, 0.0f, act};
    const KEpi* epi = (bias || act != ACT_NONE) ? &e : nullptr;
    if (R == 1 && S == 1 && stride_h == 1 && stride_w == 1 && pad_h == 0 && pad_w == 0)
        // a 1 x 1 convolution over every pixel: A is the input itself, an
        // (N H W) x C matrix -- a plain GEMM with B given as K x C rows
        return run_gemm(1, M, K, C, x, C, 0, w, C, 0, y, K, 0, stream, true, epi);
    ensure_init();
    int dev = 0;
    hipError_t he = hipGetDevice(&dev);
    if (he != hipSuccess) return fail(MKP_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(he));
    const uint16_t* zero = nullptr;
    int rc = zero_page(dev, &zero);
    if (rc != MKP_OK) return rc;
    // Channels not a multiple of 8 (or an unaligned input) would leave the
    // gathers element by element: pad the channels of the input and of the
    // filters to a multiple of 8 with zeros (the Bolt page pads kernels to
    // alignment 8) -- the same convolution with C8 channels.
    const uint16_t* xs = (const uint16_t*)x;
    const uint16_t* ws = (const uint16_t*)w;
    int64_t Cc = C;
    // the padded copies (slot 1) stay this call's until the GEMM below has
    // enqueued its launches on them
    WsLease lease1;
    if (C % 8 != 0 || !aligned16(x)) {
        hipStream_t st = (hipStream_t)stream;
        const int64_t C8 = (C + 7) & ~int64_t(7);
        const int64_t xrows = N * H * W, wrows = K * R * S;
        const size_t xbytes = ((size_t)xrows * C8 * 2 + 255) & ~size_t(255);
        if (xrows > INT_MAX || wrows > INT_MAX || R * S * C8 > INT_MAX)
            return fail(MKP_ERR_INVALID_ARG, "convolution extents exceed the 32-bit index range");
        void* buf = nullptr;
        t_call = lib().calls.load(std::memory_order_relaxed);   // the copies belong to this call's trace record
        rc = lease1.acquire(dev, st, xbytes + (size_t)wrows * C8 * 2, &buf, 1);
        if (rc != MKP_OK) return rc;
        uint16_t* xp = (uint16_t*)buf;
        uint16_t* wp = (uint16_t*)((char*)buf + xbytes);
        Library& L = lib();
        hipError_t e1 = traced(L, st, -3, 0.0, (double)xrows * (2.0 * C + 2.0 * C8), [&] {
            return launch_pack_rows((const uint16_t*)x, C, 0, xp, C8, (int)xrows, (int)C, 1, st);
        });
        if (e1 != hipSuccess) return fail(MKP_ERR_HIP, std::string("pack launch: ") + hipGetErrorString(e1));
        e1 = traced(L, st, -3, 0.0, (double)wrows * (2.0 * C + 2.0 * C8), [&] {
            return launch_pack_rows((const uint16_t*)w, C, 0, wp, C8, (int)wrows, (int)C, 1, st);
        });
        if (e1 != hipSuccess) return fail(MKP_ERR_HIP, std::string("pack launch: ") + hipGetErrorString(e1));
        xs = xp;
        ws = wp;
        Cc = C8;
    }
    const int64_t Kc = R * S * Cc;
    const KConv cv{zero, 0, (int)H, (int)W, (int)Cc, (int)S, (int)P, (int)Q, (int)stride_h, (int)stride_w,
                   (int)pad_h, (int)pad_w, (int)dil_h, (int)dil_w, (int)R};
    // GEMM view: A (N P Q) x (R S C), B the filters as K x (R S C) rows, C the NPQK output
    return run_gemm(1, M, K, Kc, xs, Kc, 0, ws, Kc, 0, y, K, 0, stream, true, epi, &cv);
}

static_assert(MKP_ACT_NONE == ACT_NONE && MKP_ACT_RELU == ACT_RELU && MKP_ACT_GELU == ACT_GELU &&
                  MKP_ACT_GELU_TANH == ACT_GELU_TANH && MKP_ACT_SILU == ACT_SILU && ACT_COUNT == 5,
              "activation codes of the C ABI and the kernels differ");

int mkp_gemm_ex(int64_t batch, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, int64_t strideA,
                const void* B, int64_t ldb, int64_t strideB, int b_layout, float* C, int64_t ldc, int64_t strideC,
                float alpha, float beta, const float* bias, int act, void* stream) {
    if (b_layout != MKP_B_KN && b_layout != MKP_B_NK) return fail(MKP_ERR_INVALID_ARG, "b_layout must be 0 or 1");
    if (act < 0 || act >= ACT_COUNT) return fail(MKP_ERR_INVALID_ARG, "unknown activation");
    if (!std::isfinite(alpha) || !std::isfinite(beta)) return fail(MKP_ERR_INVALID_ARG, "alpha and beta must be finite");
    const KEpi e{bias, alpha, beta, act};
    // the identity epilogue is the plain product
    const bool plain = alpha == 1.0f && beta == 0.0f && bias == nullptr && act == ACT_NONE;
    return run_gemm(batch, M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc, strideC, stream,
                    b_layout == MKP_B_NK, plain ? nullptr : &e);
}

int mkp_gemm_grouped(int64_t groups, int64_t M, int64_t K, const void* A, int64_t lda, const int64_t* N,
                     const void* const* B, const int64_t* ldb, float* const* C, const int64_t* ldc, void* stream) {
    return run_grouped(groups, M, K, A, lda, N, B, ldb, C, ldc, stream, false);
}

int mkp_gemm_grouped_bt(int64_t groups, int64_t M, int64_t K, const void* A, int64_t lda, const int64_t* N,
                        const void* const* B, const int64_t* ldb, float* const* C, const int64_t* ldc,
                        void* stream) {
    return run_grouped(groups, M, K, A, lda, N, B, ldb, C, ldc, stream, true);
}

int mkp_plan_describe_grouped(int64_t groups, int64_t M, int64_t K, const int64_t* N, int flags, char* buf,
                              size_t len) {
    if (groups < 1 || groups > kMaxGroups || !N) return fail(MKP_ERR_INVALID_ARG, "bad group count or widths");
    if (M < 0 || K < 0) return fail(MKP_ERR_INVALID_ARG, "negative dimension");
    std::vector<int64_t> widths;
    for (int64_t g = 0; g < groups; ++g) {
        if (N[g] < 0) return fail(MKP_ERR_INVALID_ARG, "negative dimension");
        if (N[g] > 0) widths.push_back(N[g]);
    }
    ensure_init();
    Library& L = lib();
    std::shared_ptr<const PerfTable> tab;
    SearchOptions o;
    {
        std::shared_lock<std::shared_mutex> lk(L.mu);
        tab = L.table;
        o = L.opts;
    }
    o.bt = (flags & MKP_PLAN_B_NK) != 0;
    Plan p;
    if (M > 0 && K > 0 && !widths.empty()) p = polymerize_grouped(*tab, M, K, widths, o);
    return write_out(plan_to_json(p, *tab), buf, len);
}

int mkp_plan_describe(int64_t batch, int64_t M, int64_t N, int64_t K, int align_flags, char* buf, size_t len) {
    if (batch < 0 || M < 0 || N < 0 || K < 0) return fail(MKP_ERR_INVALID_ARG, "negative dimension");
    ensure_init();
    Library& L = lib();
    std::shared_ptr<const PerfTable> tab;
    SearchOptions o;
    {
        std::shared_lock<std::shared_mutex> lk(L.mu);
        tab = L.table;
        o = L.opts;
    }
    o.bt = (align_flags & MKP_PLAN_B_NK) != 0;
    Plan p = plan_call(*tab, batch, M, N, K, o, batch <= 65535 ? L.transpose_b.load() : 0);
    return write_out(plan_to_json(p, *tab), buf, len);
}

int mkp_plan_with_table(const char* table_text, int flags, int64_t batch, int64_t M, int64_t N, int64_t K,
                        char* buf, size_t len) {
    if (!table_text) return fail(MKP_ERR_INVALID_ARG, "table text is NULL");
    if (batch < 0 || M < 0 || N < 0 || K < 0) return fail(MKP_ERR_INVALID_ARG, "negative dimension");
    PerfTable t;
    std::string err;
    if (!parse_table(table_text, t, err)) return fail(MKP_ERR_INVALID_ARG, err);
    SearchOptions o;
    o.exhaustive = (flags & MKP_PLAN_EXHAUSTIVE) != 0;
    o.bt = (flags & MKP_PLAN_B_NK) != 0;
    o.splitk_max = INT_MAX;
    {
        // the cost-model variant and the ranked-candidate option carry over
        ensure_init();
        Library& L = lib();
        std::shared_lock<std::shared_mutex> lk(L.mu);
        o.cost_mode = L.opts.cost_mode;
        o.plan_rank = L.opts.plan_rank;
        o.fuse = L.opts.fuse;
    }
    Plan p = plan_call(t, batch, M, N, K, o, batch <= 65535 ? 1 : 0);
    return write_out(plan_to_json(p, t), buf, len);
}

int mkp_load_calibration(const char* path) {
    ensure_init();
    Library& L = lib();
    std::unique_lock<std::shared_mutex> lk(L.mu);
    // NULL restores the shipped table (or the analytic stand-in without one)
    int rc = load_table_locked(L, path, path == nullptr);
    if (rc == MKP_OK) {
        L.opts.force_kernel = -1;
    }
    return rc;
}

int mkp_set_option(const char* key, const char* value) {
    if (!key || !value) return fail(MKP_ERR_INVALID_ARG, "NULL option");
    ensure_init();
    Library& L = lib();
    std::unique_lock<std::shared_mutex> lk(L.mu);
    std::string k = key, v = value;
    if (k == "force_kernel") {
        if (v.empty()) {
            L.opts.force_kernel = -1;
        } else {
            int idx = -1;
            for (size_t i = 0; i < L.table->kernels.size(); ++i)
                if (L.table->kernels[i].name == v) idx = (int)i;
            if (idx < 0) return fail(MKP_ERR_UNSUPPORTED, "no kernel named " + v + " in the active table");
            L.opts.force_kernel = idx;
        }
    } else if (k == "force_splitk") {
        int s = std::atoi(v.c_str());
        if (s < 0) return fail(MKP_ERR_INVALID_ARG, "force_splitk < 0");
        L.opts.force_splitk = s;
    } else if (k == "patterns") {
        if (v == "I") L.opts.allow_II = false;
        else if (v == "I,II" || v == "II") L.opts.allow_II = true;
        else return fail(MKP_ERR_INVALID_ARG, "patterns must be I or I,II");
    } else if (k == "transpose_b") {
        const int x = std::atoi(v.c_str());
        if (x < 0 || x > 2) return fail(MKP_ERR_INVALID_ARG, "transpose_b must be 0, 1 or 2");
        L.transpose_b.store(x);
    } else if (k == "pack_unaligned") {
        L.pack_unaligned.store(std::atoi(v.c_str()) != 0);
        return MKP_OK;
    } else if (k == "nt_stores") {
        const int x = std::atoi(v.c_str());
        if (x < 0 || x > 63) return fail(MKP_ERR_INVALID_ARG, "nt_stores must be 0 .. 63");
        L.nt_stores.store(x);
        return MKP_OK;
    } else if (k == "fused_reduce") {
        const int x = std::atoi(v.c_str());
        if (x < 0 || x > 1) return fail(MKP_ERR_INVALID_ARG, "fused_reduce must be 0 or 1");
        L.fused_reduce.store(x);
        return MKP_OK;
    } else if (k == "trace") {
        L.trace.store(std::atoi(v.c_str()) != 0);
        return MKP_OK;
    } else if (k == "exhaustive") {
        L.opts.exhaustive = std::atoi(v.c_str()) != 0;
    } else if (k == "cost_model") {
        if (v == "full") L.opts.cost_mode = COST_FULL;
        else if (v == "wave") L.opts.cost_mode = COST_WAVE;
        else if (v == "pipe") L.opts.cost_mode = COST_PIPE;
        else return fail(MKP_ERR_INVALID_ARG, "cost_model must be full, wave or pipe");
    } else if (k == "plan_rank") {
        int r = std::atoi(v.c_str());
        if (r < 0) return fail(MKP_ERR_INVALID_ARG, "plan_rank < 0");
        L.opts.plan_rank = r;
    } else if (k == "fuse_regions") {
        // one-launch Pattern II plans over kernel pairs: 0 off (the default:
        // measured no faster on the encoder linears), 1 by modelled cost
        const int x = std::atoi(v.c_str());
        if (x < 0 || x > 1) return fail(MKP_ERR_INVALID_ARG, "fuse_regions must be 0 or 1");
        L.opts.fuse = x == 1;
    } else if (k == "splitk_max") {
        int s = std::atoi(v.c_str());
        if (s < 1) return fail(MKP_ERR_INVALID_ARG, "splitk_max < 1");
        L.opts.splitk_max = s;
    } else {
        return fail(MKP_ERR_INVALID_ARG, "unknown option " + k);
    }
    clear_plans_locked(L);
    return MKP_OK;
}

int mkp_kernel_count(void) { return kernel_count(); }

const char* mkp_kernel_name(int i) {
    if (i < 0 || i >= kernel_count()) return nullptr;
    return kernel_info(i).name;
}

void mkp_cache_clear(void) {
    ensure_init();
    {
        Library& L = lib();
        std::unique_lock<std::shared_mutex> lk(L.mu);
        clear_plans_locked(L);
    }
    free_workspaces();
}

int mkp_stats(char* buf, size_t len) {
    ensure_init();
    Library& L = lib();
    std::ostringstream o;
    size_t entries;
    std::string origin;
    {
        std::shared_lock<std::shared_mutex> lk(L.mu);
        entries = L.cache.size();
        origin = L.table_origin;
    }
    o << "{\"hits\":" << L.hits.load() << ",\"misses\":" << L.misses.load() << ",\"entries\":" << entries
      << ",\"plan_us_total\":" << (double)L.plan_ns.load() / 1000.0 << ",\"launches\":" << L.launches.load()
      << ",\"table\":\"" << origin << "\"}";
    return write_out(o.str(), buf, len);
}

const char* mkp_last_error(void) { return t_last_error.c_str(); }

int mkp_trace_dump(char* buf, size_t len) {
    Library& L = lib();
    std::vector<TraceRec> recs;
    {
        std::lock_guard<std::mutex> lk(L.trace_mu);
        recs.swap(L.trace_recs);
    }
    std::ostringstream o;
    o.precision(9);
    o << "[";
    for (size_t i = 0; i < recs.size(); ++i) {
        float ms = 0.f;
        (void)hipEventSynchronize(recs[i].e1);
        (void)hipEventElapsedTime(&ms, recs[i].e0, recs[i].e1);
        (void)hipEventDestroy(recs[i].e0);
        (void)hipEventDestroy(recs[i].e1);
        const int k = recs[i].kernel;
        // -100 - d: both regions in one launch of two-tile kernel d
        const std::string name = k >= 0       ? std::string(kernel_info(k).name)
                                 : k <= -100 ? std::string(dual_info(-100 - k).first) + "+" + dual_info(-100 - k).second
                                 : k == -1   ? "splitk_reduce"
                                 : k == -2   ? "zero_fill"
                                 : k == -3   ? "pack_rows"
                                             : "transpose_b";
        if (i) o << ",";
        o << "{\"kernel\":\"" << name << "\",\"call\":" << recs[i].call << ",\"us\":" << 1000.0 * ms
          << ",\"flops\":" << recs[i].flops
          << ",\"bytes\":" << recs[i].bytes << "}";
    }
    o << "]";
    return write_out(o.str(), buf, len);
}

int mkp_calibrate(const char* path, int max_points) {
    if (!path) return fail(MKP_ERR_INVALID_ARG, "path is NULL");
    ensure_init();
    int dev = 0;
    hipError_t he = hipGetDevice(&dev);
    if (he != hipSuccess) return fail(MKP_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(he));
    hipDeviceProp_t prop;
    he = hipGetDeviceProperties(&prop, dev);
    if (he != hipSuccess) return fail(MKP_ERR_HIP, "hipGetDeviceProperties failed");
    const int cus = prop.multiProcessorCount;
    static const int grid_t[] = {1, 2, 4, 8, 16, 32, 64, 128, 256};
    int npts = (int)(sizeof(grid_t) / sizeof(grid_t[0]));
    if (max_points > 0) npts = std::min(npts, max_points);
    const int64_t kmax_cap = 16384;
    // the few-row layouts split K (below): their K is the split depth
    // times the splits, allowed up to 65536
    const int64_t kmax_split = 65536;

    // Every kernel is measured on several wave layouts: square (tm x tn
    // tiles, tm about sqrt(slots)), where each A and B tile is shared by
    // many workgroups of the wave, and one for each row class r (r tile
    // rows, at most 32 tile columns, the rest of the slots as K splits), as
    // an output of a few rows runs, where each B tile is shared by r
    // workgroups at most.
    static const int row_classes[] = {1, 2, 4, 8};
    constexpr int nclass = (int)(sizeof(row_classes) / sizeof(row_classes[0]));
    size_t a_elems = 0, b_elems = 0, c_elems = 0;   // buffers for the largest point of any kernel
    // the kernels write C (whole 128-byte rows from 256-byte aligned slices)
    // and split-K partials with the store policy of GEMM calls
    const int nt_mode = lib().nt_stores.load(std::memory_order_relaxed);
    auto store_flags = [&](int splits) {
        if (splits <= 1) return (nt_mode & 3) ? (int)KF_NT_C : 0;
        return ((nt_mode & 4) ? (int)KF_NT_C : 0) | ((nt_mode & 32) ? (int)KF_SC1_C : 0);
    };
    struct Shape { int tm, tn, s; };
    std::vector<std::array<Shape, nclass + 1>> shapes;   // [nclass]: square
    std::vector<int> occ;
    for (int i = 0; i < kernel_count(); ++i) {
        const KernelInfo& ki = kernel_info(i);
        int n = 0;
        he = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, ki.func, ki.threads, 0);
        if (he != hipSuccess || n < 1) n = 1;
        occ.push_back(n);
        const int slots = cus * n;
        std::array<Shape, nclass + 1> sh;
        for (int c = 0; c < nclass; ++c) {
            const int r = std::min(row_classes[c], slots);
            const int cols = slots / r;
            int tn = std::min(cols, 32);
            while (cols % tn) --tn;
            sh[c] = Shape{r, tn, cols / tn};
        }
        int tm = (int)std::floor(std::sqrt((double)slots));
        while (slots % tm) --tm;
        sh[nclass] = Shape{tm, slots / tm, 1};
        shapes.push_back(sh);
        for (const Shape& s : shapes.back()) {
            const int64_t M = (int64_t)s.tm * ki.uM, N = (int64_t)s.tn * ki.uN;
            const int64_t K =
                std::min<int64_t>((int64_t)grid_t[npts - 1] * ki.uK * s.s, s.s > 1 ? kmax_split : kmax_cap);
            a_elems = std::max(a_elems, (size_t)(M * K));
            b_elems = std::max(b_elems, (size_t)(K * N));
            c_elems = std::max(c_elems, (size_t)(M * N * s.s));
        }
    }
    // Operands come from a pool of at least 2 GiB (C from one of 1 GiB) whose
    // slices rotate from launch to launch, so every timed launch streams its
    // operands from HBM, as the sweeps' GEMMs do, instead of re-reading them
    // from the 256 MB last-level cache.
    auto round256 = [](size_t x) { return (x + 255) & ~size_t(255); };
    const size_t pool_ab = std::max<size_t>(size_t(2) << 30, 2 * (round256(a_elems * 2) + round256(b_elems * 2)));
    const size_t pool_c = std::max<size_t>(size_t(1) << 30, 2 * round256(c_elems * 4));
    char* pAB = nullptr;
    char* pC = nullptr;
    if (hipMalloc(&pAB, pool_ab) != hipSuccess || hipMalloc(&pC, pool_c) != hipSuccess) {
        (void)hipFree(pAB);
        return fail(MKP_ERR_OOM, "calibration buffers");
    }
    (void)launch_fill_random_bf16((uint16_t*)pAB, (int64_t)(pool_ab / 2), 12345u, nullptr);
    (void)hipMemset(pC, 0, pool_c);
    (void)hipDeviceSynchronize();
    uint16_t* dB = (uint16_t*)pAB;   // probes below use the pool directly
    float* dC = (float*)pC;
    int64_t rotation = 0;
    // point a, for an M x K by K x N product, at the next slices of the pools
    auto next_operands = [&](KArgs& a) {
        const size_t fa = round256((size_t)a.M * a.K * 2), fb = round256((size_t)a.K * a.N * 2);
        const size_t fc = round256((size_t)a.M * a.N * 4 * std::max(a.splits, 1));
        const size_t nab = std::max<size_t>(1, pool_ab / (fa + fb)), nc = std::max<size_t>(1, pool_c / fc);
        const size_t i = (size_t)rotation++;
        char* base = pAB + (i % nab) * (fa + fb);
        a.A = (const uint16_t*)base;
        a.B = (const uint16_t*)(base + fa);
        a.C = (float*)(pC + (i % nc) * fc);
    };

    PerfTable t;
    t.cus = cus;
    t.splits = {1, 2, 3, 4, 5, 6, 8, 12, 16, 24, 32};
    t.row_classes.assign(row_classes, row_classes + nclass);
    hipError_t err = hipSuccess;
    // launch overhead: a one-workgroup kernel back to back
    t.launch_us = time_launches([&] { return launch_zero_fill(dC, 1, 0, 1, 1, 1, nullptr); }, 20, 200, &err);
    // split-K reduction: fixed cost and bandwidth fitted to two partial
    // volumes, in the cost model's byte count (2s+1)*4*m*n
    {
        struct P { int s, m, n; };
        const P pa{2, 16, 4096}, pb{8, 256, 8192};
        float* W = nullptr;
        if (hipMalloc(&W, (size_t)pb.s * pb.m * pb.n * 4) == hipSuccess) {
            (void)hipMemset(W, 0, (size_t)pb.s * pb.m * pb.n * 4);
            float* Cr = nullptr;
            if (hipMalloc(&Cr, (size_t)pb.m * pb.n * 4) == hipSuccess) {
                auto run = [&](const P& q) {
                    return time_launches([&] {
                        return launch_splitk_reduce(W, q.s, (int64_t)q.m * q.n, 0, q.n, Cr, q.n, 0, q.m, q.n, 1, 1,
                                                    nullptr);
                    }, 20, 50, &err);
                };
                const double ta = run(pa), tb = run(pb);
                const double ba = (2.0 * pa.s + 1) * 4.0 * pa.m * pa.n, bb = (2.0 * pb.s + 1) * 4.0 * pb.m * pb.n;
                const double bw = (bb - ba) / std::max(tb - ta, 0.1);   // bytes per us
                t.red_gbps = bw / 1e3;
                t.red_launch_us = std::max(ta - ba / bw, 0.0);
                (void)hipFree(Cr);
            }
            (void)hipFree(W);
        }
    }
    // transpose of a K x N B into N x K: fixed cost and bandwidth fitted to
    // two sizes, in the cost model's byte count 4*K*N; source and target
    // rotate through the pool like the kernels' operands
    {
        int64_t slot = 0;
        auto run = [&](int K, int N) {
            const size_t bytes = round256((size_t)K * N * 2);
            const size_t nslots = std::max<size_t>(2, pool_ab / bytes);
            return time_launches([&] {
                char* src = pAB + (size_t)(slot % nslots) * bytes;
                char* dst = pAB + (size_t)((slot + 1) % nslots) * bytes;
                slot += 2;
                return launch_transpose_bf16((const uint16_t*)src, N, 0, (uint16_t*)dst, K, 0, K, N, 1, true, nullptr);
            }, 10, 30, &err);
        };
        const double ta = run(768, 768), tb = run(4096, 4096);
        const double ba = 4.0 * 768 * 768, bb = 4.0 * 4096 * 4096;
        const double bw = (bb - ba) / std::max(tb - ta, 0.1);   // bytes per us
        t.tr_gbps = bw / 1e3;
        t.tr_launch_us = std::max(ta - ba / bw, 0.0);
    }
    for (int i = 0; i < kernel_count() && err == hipSuccess; ++i) {
        const KernelInfo& ki = kernel_info(i);
        TableKernel k;
        k.name = ki.name;
        k.uM = ki.uM;
        k.uN = ki.uN;
        k.uK = ki.uK;
        k.wg_per_cu = occ[i];
        k.lib_index = i;
        k.bt = ki.bt;
        k.by_rows.assign(nclass, Curves{});
        for (int layout = 0; layout <= nclass && err == hipSuccess; ++layout) {
            const Shape s = shapes[i][layout];
            Curves square;
            Curves& cv = layout < nclass ? k.by_rows[layout] : square;
            auto& pts = cv.pts;
            auto& tail = cv.tail;
            auto& tailx = cv.tailx;
            for (int p = 0; p < npts; ++p) {
                const int tt = grid_t[p];
                const int64_t K = (int64_t)tt * ki.uK * s.s;
                if (K > (s.s > 1 ? kmax_split : kmax_cap)) break;
                KArgs a{};
                a.M = s.tm * ki.uM;
                a.N = s.tn * ki.uN;
                a.K = (int)K;
                a.lda = K;
                a.ldb = ki.bt ? a.K : a.N;
                a.ldc = a.N;
                a.tiles_m = s.tm;
                a.tiles_n = s.tn;
                a.steps_per_split = tt;
                a.splits = s.s;
                a.sCsplit = s.s > 1 ? (int64_t)a.M * a.N : 0;   // each split's partial tile
                a.batch = 1;
                a.flags = KF_VEC_A | KF_VEC_B | KF_VEC_C | store_flags(s.s);
                const dim3 grid((unsigned)(s.tm * s.tn * s.s));
                // single-launch time, then enough repetitions for ~2 ms
                auto launch = [&] {
                    next_operands(a);
                    return ki.launch(a, grid, nullptr);
                };
                double us = time_launches(launch, 3, 3, &err);
                if (err != hipSuccess) break;
                int reps = (int)std::min(200.0, std::max(5.0, 2000.0 / std::max(us, 1.0)));
                // the median of three timed runs (a clock or power-state
                // change can upset one of them)
                double run[3];
                for (int r = 0; r < 3 && err == hipSuccess; ++r) run[r] = time_launches(launch, r ? 3 : 20, reps, &err);
                if (err != hipSuccess) break;
                std::sort(run, run + 3);
                us = run[1];
                pts.emplace_back((double)tt, std::max(us - t.launch_us, 0.05));
            }
            // partial last wave, at 16 K steps, relative to a full wave of the
            // same depth: a wave filling a fraction f of the slots on its own
            // (tail), and the time f adds after one full wave (tailx)
            const int t_ref = 16;
            double g_ref = 0;
            for (auto& pt : pts)
                if (pt.first == t_ref) g_ref = pt.second;
            if (err == hipSuccess && g_ref > 0) {
                static const double fills[] = {1.0 / 16, 1.0 / 8, 1.0 / 4, 1.0 / 2, 3.0 / 4};
                const int slots = s.tm * s.tn * s.s;
                int prev_tn = 0;
                for (double f : fills) {
                    const int tn = std::max(1, (int)std::lround(f * s.tn));
                    if (tn == prev_tn || tn >= s.tn) continue;
                    prev_tn = tn;
                    double us[2];
                    for (int after = 0; after < 2 && err == hipSuccess; ++after) {
                        const int cols = tn + (after ? s.tn : 0);
                        KArgs a{};
                        a.M = s.tm * ki.uM;
                        a.N = cols * ki.uN;
                        a.K = t_ref * ki.uK * s.s;
                        a.lda = a.K;
                        a.ldb = ki.bt ? a.K : a.N;
                        a.ldc = a.N;
                        a.tiles_m = s.tm;
                        a.tiles_n = cols;
                        a.steps_per_split = t_ref;
                        a.splits = s.s;
                        a.sCsplit = s.s > 1 ? (int64_t)a.M * a.N : 0;
                        a.batch = 1;
                        a.flags = KF_VEC_A | KF_VEC_B | KF_VEC_C | store_flags(s.s);
                        const dim3 grid((unsigned)(s.tm * cols * s.s));
                        us[after] = time_launches(
                            [&] {
                                next_operands(a);
                                return ki.launch(a, grid, nullptr);
                            },
                            20, 50, &err);
                    }
                    if (err != hipSuccess) break;
                    const double fill = (double)(s.tm * tn * s.s) / slots;
                    auto clamp = [](double r) { return std::min(1.0, std::max(0.02, r)); };
                    tail.emplace_back(fill, clamp(std::max(us[0] - t.launch_us, 0.05) / g_ref));
                    tailx.emplace_back(fill, clamp((us[1] - t.launch_us - g_ref) / g_ref));
                }
            }
            if (layout == nclass) {
                k.pts = square.pts;
                k.tail = square.tail;
                k.tailx = square.tailx;
            }
        }
        t.kernels.push_back(k);
        std::fprintf(stderr, "[calibrate] %d/%d %s\n", i + 1, kernel_count(), ki.name);
        std::fflush(stderr);
    }
    // sustained ceilings: MFMA on random operands, streaming copy
    if (err == hipSuccess) {
        const int blocks = cus, iters = 256;
        const double us = time_launches([&] { return launch_mfma_probe(dC, blocks, iters, nullptr); }, 5, 10, &err);
        t.mfma_tflops = (double)blocks * 4 * 64.0 * iters * 32768.0 / us / 1e6;
    }
    if (err == hipSuccess) {
        // copy between the two halves of the operand pool, up to 1 GB each
        // way (well beyond the 256 MB MALL)
        const int64_t half = (int64_t)(pool_ab / 2);
        const int64_t bytes = std::min<int64_t>(half, int64_t(1) << 30) & ~int64_t(15);
        char* base = (char*)dB;
        const double us = time_launches(
            [&] { return launch_copy_probe(base, base + (half & ~int64_t(255)), bytes, cus * 8, nullptr); }, 3, 10, &err);
        t.hbm_gbps = 2.0 * (double)bytes / us / 1e3;
    }
    if (err == hipSuccess) {
        // read-only streaming of up to 1 GB, alternating between the two
        // halves of the pool (each launch reads data the last one did not)
        const int64_t half = (int64_t)(pool_ab / 2) & ~int64_t(255);
        const int64_t bytes = std::min<int64_t>(half, int64_t(1) << 30) & ~int64_t(15);
        const int blocks = cus * 8;
        char* base = (char*)dB;
        int flip = 0;
        const double us = time_launches(
            [&] { return launch_read_probe(base + (flip++ & 1) * half, bytes, (uint32_t*)dC, blocks, nullptr); }, 3, 10,
            &err);
        t.hbm_read_gbps = (double)bytes / us / 1e3;
    }
    (void)hipDeviceSynchronize();
    (void)hipFree(pAB);
    (void)hipFree(pC);
    if (err != hipSuccess) return fail(MKP_ERR_HIP, std::string("calibration launch: ") + hipGetErrorString(err));
    {
        // the library's one-launch kernel pairs, written out with the table
        std::string berr;
        if (!bind_table(t, berr)) return fail(MKP_ERR_UNSUPPORTED, "calibrated table: " + berr);
    }

    std::string text = "# measured by mkp_calibrate on " + std::string(prop.name) + " (" +
                       std::string(prop.gcnArchName) + "), " + std::to_string(cus) + " CUs\n" + table_to_text(t);
    {
        std::ofstream f(path);
        if (!f) return fail(MKP_ERR_INVALID_ARG, std::string("cannot write ") + path);
        f << text;
    }
    Library& L = lib();
    std::unique_lock<std::shared_mutex> lk(L.mu);
    L.table = std::make_shared<const PerfTable>(std::move(t));
    L.table_origin = path;
    L.opts.force_kernel = -1;
    clear_plans_locked(L);
    return MKP_OK;
}

}  // extern "C"
