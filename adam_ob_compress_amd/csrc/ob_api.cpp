// ob_api.cpp -- host runtime and C ABI of libobadam.so (declarations and contracts in ob_adam.h).
//
// The host side only validates arguments, owns the plan's small device tables and enqueues kernels
// on the caller's stream; every step of the optimizer runs in ob_kernels.hip.
#include "ob_adam.h"
#include "ob_internal.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <new>
#include <vector>

struct ob_plan_s {
    int device = 0;
    int64_t n = 0;
    int32_t K = 0;
    int64_t* d_chunk_off = nullptr;
    double* d_partials = nullptr;  // one per pass-1 block
    int64_t p1_max = 0;            // most pass-1 blocks in one chunk
    bool off128 = false;           // every chunk offset is a multiple of 128 elements
    // plans with more than kFinalizeAt pass-1 blocks in a chunk: per-chunk sums and the identity table
    double* d_chunk_sums = nullptr;  // [K]
    int32_t* d_ident = nullptr;      // [K + 1]: 0, 1, ..., K
    // LAMB: per-block sums of p^2 (written by pass 1, the dense step and the worker update, each over
    // its own block table) and of u^2 (compressed pass 2, the dense step, the worker update); each is
    // sized for the largest table that writes it, and every launch that writes them is checked
    // against these sizes on the host (lamb_fits)
    double* d_partials_w = nullptr;
    double* d_partials_u = nullptr;
    int64_t n_partials_w = 0;
    int64_t n_partials_u = 0;

    // diagnostics (off until ob_plan_set_diagnostics): workspaces and the caller's output arrays
    double* d_partials_e = nullptr;    // one per pass-1 block
    uint32_t* d_partials_b = nullptr;  // one per compressed-pass-2 block
    double* diag_err_sumsq = nullptr;
    unsigned long long* diag_plus = nullptr;

    // Chunk groups of the compressed step's two passes.  Pass 2 re-reads g and err, which pass 1 has
    // just read; run over consecutive chunks whose pass-1 bytes about fit in the GPU's last-level cache
    // (the Infinity Cache, 256 MB on MI355X), pass 1 then pass 2 per group serves most of that re-read
    // from the cache instead of HBM.  groups[w]: the groups when pass 1 reads w bytes per element (g
    // and err: 4, 6 or 8); one group of all chunks when grouping is off.  whole: one group of all
    // chunks, for 1-bit LAMB (its pass 1 also reads p, and groups measured no faster there).
    int64_t group_bytes = 0;
    std::vector<ob::ChunkGroup> groups[9];
    std::vector<ob::ChunkGroup> whole;

    // block tables, one per kernel kind (kTables)
    struct Table {
        int64_t block_elems = 0;
        int64_t n_items = 0;
        ob::Item* d_items = nullptr;
        int32_t* d_first = nullptr;
    } t[4];

    // kernel timing
    bool timing = false;
    struct Rec {
        int kernel;
        hipEvent_t a, b;
        bool owns_a;   // false: a is the previous record's b (a chained launch), pooled with that record
    };
    std::vector<Rec> pending;
    std::vector<hipEvent_t> pool;
    double total_ms[OB_KERNEL_COUNT] = {};
    int64_t launches[OB_KERNEL_COUNT] = {};

    ob::PlanDev dev(int table) const
    {
        ob::PlanDev pd;
        pd.items = t[table].d_items;
        pd.chunk_first = t[table].d_first;
        pd.p1_first = t[0].d_first;
        pd.chunk_off = d_chunk_off;
        pd.partials = d_partials;
        pd.partials_w = d_partials_w;
        pd.w_first = nullptr;
        pd.partials_u = d_partials_u;
        pd.u_first = nullptr;
        const bool diag = diag_err_sumsq != nullptr;
        pd.partials_e = diag ? d_partials_e : nullptr;
        pd.partials_b = diag ? d_partials_b : nullptr;
        pd.n = n;
        pd.n_items = t[table].n_items;
        pd.K = K;
        pd.item0 = 0;
        return pd;
    }
};

namespace {

constexpr int64_t kMaxBlockElems = int64_t(1) << 20;

// Chunks with more pass-1 partials than this get one sum per chunk (a one-block-per-chunk kernel)
// before pass 2; below it every pass-2 block adds its chunk's partials itself, with no extra launch.
// Measured: at 1,761 partials (BERT-base's embedding) the in-block reduction is still the faster; the
// extra launch is for chunks so large that every block re-adding their partials would dominate.
constexpr int64_t kFinalizeAt = 16 * ob::kBlock;

// Pass-1 bytes per chunk group (the compressed step's passes run group by group).  Measured on MI355X
// (interleaved A/B in one process, outputs bit-identical): 320 MB groups took the Llama-2-7B-sized
// step (6.7G elements, bf16 g) from 40.8 to 37.9 ms, the GPT-2-1.5B-sized one from 8.75 to 8.35 ms and
// the BERT-base-sized one from 0.705 to 0.672 ms; 192 and 400 MB were 1-2% slower than 320, 64 MB (one
// chunk per group) no faster than no groups at all, and the same groups with nontemporal pass-1 loads
// (which do not stay in the cache) slower than no groups.
// OB_GROUP_BYTES overrides (0 = one launch per pass).
constexpr int64_t kGroupBytes = int64_t(320) << 20;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Make the plan's device current for the duration of a call.
struct DeviceGuard {
    int prev = -1;
    bool ok = true;
    explicit DeviceGuard(int dev)
    {
        if (hipGetDevice(&prev) != hipSuccess) {
            ok = false;
            return;
        }
        if (prev != dev && hipSetDevice(dev) != hipSuccess) ok = false;
    }
    ~DeviceGuard()
    {
        int cur = -1;
        if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
    }
};

// Block tables by kernel kind.  Elements per block (from sweeps of 1-128 tiles of 1024 on MI355X):
//   pass 1 (sums of squares): large blocks, so a chunk has few partial sums: enough blocks to fill
//     256 CUs several times over, whole tiles, at most 24 tiles (measured: with 64-tile pass-1 blocks
//     the pass 2 that follows ran 2% slower on 1.5G- and 6.7G-element buffers, 0.5% on the latter's
//     whole step; 8-tile blocks slowed pass 1 itself);
//   compressed pass 2: 4 tiles;  dense step: 2 tiles;  server pass 2 and unpack: 8 tiles.
// Environment overrides for tuning sweeps (multiples of 1024): OB_BLOCK_ELEMS, OB_BLOCK_ELEMS2,
// OB_BLOCK_ELEMS_DENSE, OB_BLOCK_ELEMS_SERVER.
enum { T_PASS1 = 0, T_COMPRESS = 1, T_DENSE = 2, T_SERVER = 3, kTables = 4 };

int64_t env_block_elems(const char* name)
{
    if (const char* env = std::getenv(name)) {
        const long long v = std::atoll(env);
        if (v >= ob::kTile && v <= kMaxBlockElems && v % ob::kTile == 0) return v;
    }
    return 0;
}

int64_t choose_block_elems(int64_t n, int table)
{
    static const char* const env[kTables] = {"OB_BLOCK_ELEMS", "OB_BLOCK_ELEMS2", "OB_BLOCK_ELEMS_DENSE",
                                             "OB_BLOCK_ELEMS_SERVER"};
    static const int64_t tiles[kTables] = {0, 4, 2, 8};
    if (const int64_t e = env_block_elems(env[table])) return e;
    if (table != T_PASS1) return tiles[table] * ob::kTile;
    const int64_t target_blocks = 8192;
    int64_t e = (n + target_blocks - 1) / target_blocks;
    e = (e + ob::kTile - 1) / ob::kTile * ob::kTile;
    return std::min<int64_t>(std::max<int64_t>(e, 4 * ob::kTile), 24 * ob::kTile);
}

int64_t group_budget()
{
    if (const char* env = std::getenv("OB_GROUP_BYTES")) return std::max<long long>(0, std::atoll(env));
    return kGroupBytes;
}

// The chunk groups a compressed step runs its two passes over: by the bytes per element pass 1 reads
// (g and the error buffer), or one group for 1-bit LAMB.
const std::vector<ob::ChunkGroup>& step_groups(ob_plan p, int g_dtype, int err_dtype, int lamb)
{
    if (lamb) return p->whole;
    return p->groups[(g_dtype == OB_BF16 ? 2 : 4) + (err_dtype == OB_F32 ? 4 : 2)];
}

// A launch over blocks [i0, i0 + count) of the view's table.
ob::PlanDev group_view(ob::PlanDev pd, int32_t i0, int32_t count)
{
    pd.item0 = i0;
    pd.n_items = count;
    return pd;
}

void free_plan(ob_plan p)
{
    if (!p) return;
    for (auto& r : p->pending) {
        if (r.owns_a) (void)hipEventDestroy(r.a);   // a chained record's a is the previous record's b
        (void)hipEventDestroy(r.b);
    }
    for (auto e : p->pool) (void)hipEventDestroy(e);
    for (auto& t : p->t) {
        if (t.d_items) (void)hipFree(t.d_items);
        if (t.d_first) (void)hipFree(t.d_first);
    }
    if (p->d_chunk_off) (void)hipFree(p->d_chunk_off);
    if (p->d_partials) (void)hipFree(p->d_partials);
    if (p->d_partials_w) (void)hipFree(p->d_partials_w);
    if (p->d_partials_u) (void)hipFree(p->d_partials_u);
    if (p->d_partials_e) (void)hipFree(p->d_partials_e);
    if (p->d_chunk_sums) (void)hipFree(p->d_chunk_sums);
    if (p->d_ident) (void)hipFree(p->d_ident);
    if (p->d_partials_b) (void)hipFree(p->d_partials_b);
    delete p;
}

hipEvent_t take_event(ob_plan p)
{
    if (!p->pool.empty()) {
        hipEvent_t e = p->pool.back();
        p->pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    // Timing-only events: no system-scope fence when an event completes, so recording one does not
    // write back and invalidate the caches in front of the next kernel (a plain event cost a
    // BERT-base step about 14 us, this one about 8).  Elapsed times stay exact; the events are never
    // used to order memory.
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
    return e;
}

// Enqueue one kernel via `launch`, bracketed by events when timing is on.  chain != nullptr: launches
// of one call that follow each other on the stream with nothing in between share events -- a launch
// starts at the event that ended the previous one (*chain, if set) and leaves its own end event in
// *chain -- so a call with many launches (the compressed step's chunk groups) records one event per
// launch instead of two.
template <class F>
ob_status timed(ob_plan p, int kernel, hipStream_t s, F&& launch, hipEvent_t* chain = nullptr)
{
    hipEvent_t a = nullptr, b = nullptr;
    bool owns_a = true;
    if (p && p->timing) {
        if (chain && *chain) {
            a = *chain;
            owns_a = false;
        } else {
            a = take_event(p);
        }
        b = take_event(p);
        if (a && b && owns_a) (void)hipEventRecord(a, s);
    }
    (void)hipGetLastError();  // clear a stale error so the check below sees this launch only
    const hipError_t err = launch();
    if (a && b) {
        (void)hipEventRecord(b, s);
        p->pending.push_back({kernel, a, b, owns_a});
        if (chain) *chain = b;
    } else {
        if (a && owns_a) p->pool.push_back(a);
        if (b) p->pool.push_back(b);
        if (chain) *chain = nullptr;
    }
    return err == hipSuccess ? OB_OK : OB_ERR_HIP;
}

ob_status drain_timing(ob_plan p)
{
    ob_status st = OB_OK;
    for (auto& r : p->pending) {
        float ms = 0.0f;
        if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess)
            st = OB_ERR_HIP;
        else {
            p->total_ms[r.kernel] += ms;
            p->launches[r.kernel] += 1;
        }
        if (r.owns_a) p->pool.push_back(r.a);
        p->pool.push_back(r.b);
    }
    p->pending.clear();
    return st;
}

// gradient / packed-input types
bool valid_dtype(int d) { return d == OB_F32 || d == OB_BF16; }

ob::DenseParams dense_params(const ob_hparams* hp)
{
    ob::DenseParams dp;
    dp.lr = hp->lr;
    dp.beta1 = hp->beta1;
    dp.one_m_beta1 = 1.0 - static_cast<double>(hp->beta1);
    dp.beta2 = hp->beta2;
    dp.one_m_beta2 = 1.0 - static_cast<double>(hp->beta2);
    dp.eps = hp->eps;
    dp.bias_correction = hp->bias_correction ? 1 : 0;
    dp.bc1 = 1.0;
    dp.bc2 = 1.0;
    if (hp->bias_correction) {
        dp.bc1 = 1.0 - std::pow(static_cast<double>(hp->beta1), static_cast<double>(hp->step));
        dp.bc2 = 1.0 - std::pow(static_cast<double>(hp->beta2), static_cast<double>(hp->step));
    }
    return dp;
}
// error-buffer storage formats
bool valid_err_dtype(int d) { return d == OB_F32 || d == OB_BF16 || d == OB_F16; }

ob_status check_grad(const void* g, int dt)
{
    if (!valid_dtype(dt)) return OB_ERR_DTYPE;
    if (!g) return OB_ERR_ARG;
    return aligned(g, dt == OB_BF16 ? 8 : 16) ? OB_OK : OB_ERR_ALIGN;
}

}  // namespace

// LAMB launches write one double per block of their table into the plan's p^2 and/or u^2 workspaces;
// refuse a launch whose table has more blocks than the workspace it writes holds (cannot happen with
// the sizes ob_plan_create takes, whatever block sizes the tuning knobs choose; kept as a guard).
static bool lamb_fits(ob_plan p, int table, bool writes_w, bool writes_u)
{
    const int64_t k = p->t[table].n_items;
    return (!writes_w || k <= p->n_partials_w) && (!writes_u || k <= p->n_partials_u);
}

extern "C" {

const char* ob_status_str(ob_status s)
{
    switch (s) {
    case OB_OK: return "ok";
    case OB_ERR_ARG: return "invalid argument";
    case OB_ERR_ALIGN: return "misaligned pointer or chunk boundary";
    case OB_ERR_DTYPE: return "unknown dtype";
    case OB_ERR_HIP: return "HIP runtime error";
    case OB_ERR_OOM: return "device allocation failed";
    case OB_ERR_SIZE: return "problem too large for the no-allocation entry point's static buffer";
    }
    return "unknown status";
}

}  // extern "C"

namespace {

// ob_plan_create's body.  p: the plan being built, owned here until it is handed out in *out (every
// return that fails frees it first), so that the caller can free it if an exception escapes.
ob_status plan_create(int64_t n, int64_t chunk_size, const int64_t* chunk_offsets, int64_t n_chunks, ob_plan* out,
                      ob_plan& p)
{
    if (!out) return OB_ERR_ARG;
    *out = nullptr;
    if (n < 0) return OB_ERR_ARG;

    // chunk table (host)
    std::vector<int64_t> off;
    if (chunk_offsets == nullptr) {
        if (chunk_size <= 0) return OB_ERR_ARG;
        if (n > 0) {
            const int64_t K = (n + chunk_size - 1) / chunk_size;
            if (K > 1 && chunk_size % 64 != 0) return OB_ERR_ALIGN;
            if (K > INT32_MAX - 1) return OB_ERR_ARG;
            off.resize(static_cast<size_t>(K) + 1);
            for (int64_t c = 0; c < K; ++c) off[c] = c * chunk_size;
            off[K] = n;
        } else {
            off.push_back(0);
        }
    } else {
        if (n_chunks < 0 || n_chunks > INT32_MAX - 1) return OB_ERR_ARG;
        if (n > 0 && n_chunks < 1) return OB_ERR_ARG;
        off.assign(chunk_offsets, chunk_offsets + n_chunks + 1);
        if (off[0] != 0 || off.back() != n) return OB_ERR_ARG;
        for (int64_t c = 0; c < n_chunks; ++c)
            if (off[c + 1] <= off[c]) return OB_ERR_ARG;
        for (int64_t c = 1; c < n_chunks; ++c)
            if (off[c] % 64 != 0) return OB_ERR_ALIGN;
    }
    const int64_t K = static_cast<int64_t>(off.size()) - 1;

    p = new (std::nothrow) ob_plan_s;
    if (!p) return OB_ERR_OOM;
    p->n = n;
    p->K = static_cast<int32_t>(K);

    // block tables: consecutive blocks per chunk, checked against what the kernels assume before any
    // of them reaches the device
    std::vector<ob::Item> items[kTables];
    std::vector<int32_t> first[kTables];
    for (int pass = 0; pass < kTables; ++pass) {
        ob_plan_s::Table& t = p->t[pass];
        t.block_elems = choose_block_elems(n, pass);
        if (!ob::build_block_table(off, t.block_elems, items[pass], first[pass]) ||
            ob::check_block_table(off, t.block_elems, items[pass], first[pass]) != nullptr) {
            delete p;
            return OB_ERR_ARG;
        }
        t.n_items = static_cast<int64_t>(items[pass].size());
    }
    for (int64_t c = 0; c < K; ++c)
        p->p1_max = std::max<int64_t>(p->p1_max, first[T_PASS1][c + 1] - first[T_PASS1][c]);
    p->off128 = std::all_of(off.begin(), off.end() - 1, [](int64_t o) { return o % 128 == 0; });
    // chunk groups (none while any chunk needs its sums formed by a launch of their own)
    p->group_bytes = group_budget();
    const bool grouping = p->group_bytes > 0 && p->p1_max <= kFinalizeAt;
    for (int w = 4; w <= 8; w += 2) {
        const int64_t max_elems = grouping ? std::max<int64_t>(1, p->group_bytes / w) : 0;
        ob::build_chunk_groups(off, first[T_PASS1], first[T_COMPRESS], max_elems, p->groups[w]);
        if (ob::check_chunk_groups(off, first[T_PASS1], first[T_COMPRESS], max_elems, p->groups[w]) != nullptr) {
            delete p;
            return OB_ERR_ARG;
        }
    }
    ob::build_chunk_groups(off, first[T_PASS1], first[T_COMPRESS], 0, p->whole);

    if (hipGetDevice(&p->device) != hipSuccess) {
        delete p;
        return OB_ERR_HIP;
    }
    if (n > 0) {
        auto fail = [&](hipError_t e) {
            free_plan(p);
            return e == hipErrorOutOfMemory ? OB_ERR_OOM : OB_ERR_HIP;
        };
        hipError_t e;
        for (int pass = 0; pass < kTables; ++pass) {
            ob_plan_s::Table& t = p->t[pass];
            if ((e = hipMalloc(&t.d_items, items[pass].size() * sizeof(ob::Item))) != hipSuccess) return fail(e);
            if ((e = hipMalloc(&t.d_first, first[pass].size() * sizeof(int32_t))) != hipSuccess) return fail(e);
            if ((e = hipMemcpy(t.d_items, items[pass].data(), items[pass].size() * sizeof(ob::Item),
                               hipMemcpyHostToDevice)) != hipSuccess)
                return fail(e);
            if ((e = hipMemcpy(t.d_first, first[pass].data(), first[pass].size() * sizeof(int32_t),
                               hipMemcpyHostToDevice)) != hipSuccess)
                return fail(e);
        }
        if ((e = hipMalloc(&p->d_partials, items[0].size() * sizeof(double))) != hipSuccess) return fail(e);
        if (p->p1_max > kFinalizeAt) {
            std::vector<int32_t> ident(static_cast<size_t>(K) + 1);
            for (int64_t c = 0; c <= K; ++c) ident[c] = static_cast<int32_t>(c);
            if ((e = hipMalloc(&p->d_chunk_sums, static_cast<size_t>(K) * sizeof(double))) != hipSuccess) return fail(e);
            if ((e = hipMalloc(&p->d_ident, ident.size() * sizeof(int32_t))) != hipSuccess) return fail(e);
            if ((e = hipMemcpy(p->d_ident, ident.data(), ident.size() * sizeof(int32_t), hipMemcpyHostToDevice)) !=
                hipSuccess)
                return fail(e);
        }
        const size_t nw = std::max({items[T_PASS1].size(), items[T_COMPRESS].size(), items[T_DENSE].size()});
        const size_t nu = std::max(items[T_COMPRESS].size(), items[T_DENSE].size());
        if ((e = hipMalloc(&p->d_partials_w, nw * sizeof(double))) != hipSuccess) return fail(e);
        if ((e = hipMalloc(&p->d_partials_u, nu * sizeof(double))) != hipSuccess) return fail(e);
        p->n_partials_w = static_cast<int64_t>(nw);
        p->n_partials_u = static_cast<int64_t>(nu);
        if ((e = hipMalloc(&p->d_chunk_off, off.size() * sizeof(int64_t))) != hipSuccess) return fail(e);
        if ((e = hipMemcpy(p->d_chunk_off, off.data(), off.size() * sizeof(int64_t), hipMemcpyHostToDevice)) !=
            hipSuccess)
            return fail(e);
    }
    *out = p;
    return OB_OK;
}

}  // namespace

extern "C" {

ob_status ob_plan_create(int64_t n, int64_t chunk_size, const int64_t* chunk_offsets, int64_t n_chunks,
                         ob_plan* out)
{
    ob_plan p = nullptr;
    try {
        return plan_create(n, chunk_size, chunk_offsets, n_chunks, out, p);
    } catch (...) {
        // a host allocation of the tables or groups failed (the only exceptions here): free what the
        // plan holds so far and report it like a failed device allocation
        if (p) free_plan(p);
        if (out) *out = nullptr;
        return OB_ERR_OOM;
    }
}

ob_status ob_plan_destroy(ob_plan plan)
try {
    if (!plan) return OB_ERR_ARG;
    DeviceGuard g(plan->device);
    free_plan(plan);
    return OB_OK;
} catch (...) {
    return OB_ERR_OOM;  // host allocation failures are the only exceptions here
}

int64_t ob_plan_num_elements(ob_plan plan) { return plan ? plan->n : -1; }
int64_t ob_plan_num_chunks(ob_plan plan) { return plan ? plan->K : -1; }
int64_t ob_plan_num_blocks(ob_plan plan) { return plan ? plan->t[T_COMPRESS].n_items : -1; }
int64_t ob_plan_block_elems(ob_plan plan) { return plan ? plan->t[T_COMPRESS].block_elems : -1; }
int64_t ob_plan_num_groups(ob_plan plan, ob_dtype g_dtype, ob_dtype err_dtype, int32_t lamb)
{
    if (!plan || !valid_dtype(g_dtype) || !valid_err_dtype(err_dtype)) return -1;
    return static_cast<int64_t>(step_groups(plan, g_dtype, err_dtype, lamb).size());
}

ob_status ob_adam_warmup_step(ob_plan plan, const void* g, ob_dtype g_dtype, float* m, float* v, float* p,
                              const ob_hparams* hp, hipStream_t stream)
try {
    if (!plan || !hp) return OB_ERR_ARG;
    if (!valid_dtype(g_dtype)) return OB_ERR_DTYPE;
    if (plan->n == 0) return OB_OK;
    if (ob_status st = check_grad(g, g_dtype)) return st;
    if (!m || !v || !p) return OB_ERR_ARG;
    if (!aligned(m, 16) || !aligned(v, 16) || !aligned(p, 16)) return OB_ERR_ALIGN;
    if (hp->bias_correction && hp->step < 1) return OB_ERR_ARG;

    const ob::DenseParams dp = dense_params(hp);
    DeviceGuard guard(plan->device);
    if (!guard.ok) return OB_ERR_HIP;
    const ob::PlanDev pd = plan->dev(T_DENSE);
    const int bf = g_dtype == OB_BF16;
    return timed(plan, OB_KERNEL_DENSE, stream,
                 [&] { return ob::launch_dense(pd, g, bf, m, v, p, 0, dp, stream); });
} catch (...) {
    return OB_ERR_OOM;  // host allocation failures are the only exceptions here
}

}  // extern "C"

namespace {

// Arguments of the compressed step after the plan (or n) checks: dtypes already valid, n > 0.
ob_status check_compress_args(const void* g, ob_dtype g_dtype, const void* err, ob_dtype err_dtype,
                              const float* m, const float* v, const float* p, const uint32_t* words_out,
                              const float* scales_out, const int8_t* signs_out, const uint64_t* nonfinite_out,
                              const ob_hparams* hp)
{
    if (ob_status st = check_grad(g, g_dtype)) return st;
    if (!err || !m || !v || !p || !words_out || !scales_out) return OB_ERR_ARG;
    if (!aligned(err, err_dtype == OB_F32 ? 16 : 8)) return OB_ERR_ALIGN;
    if (!aligned(m, 16) || !aligned(v, 16) || !aligned(p, 16)) return OB_ERR_ALIGN;
    if (!aligned(words_out, 4) || !aligned(scales_out, 4)) return OB_ERR_ALIGN;
    if (signs_out && !aligned(signs_out, 4)) return OB_ERR_ALIGN;
    if (nonfinite_out && !aligned(nonfinite_out, 8)) return OB_ERR_ALIGN;
    if (hp->ef_mode != OB_EF_PLAIN && hp->ef_mode != OB_EF_EMA) return OB_ERR_ARG;
    if (hp->err_rounding != OB_ROUND_NEAREST && hp->err_rounding != OB_ROUND_STOCHASTIC) return OB_ERR_ARG;
    if (hp->err_rounding == OB_ROUND_STOCHASTIC && err_dtype == OB_F32) return OB_ERR_ARG;
    return OB_OK;
}

// nt: nontemporal loads, for a pass 1 over all chunks at once (no chunk groups)
hipError_t sumsq_by_format(ob_dtype err_dtype, const ob::PlanDev& pd1, const void* g, int bf, const void* err,
                           float clip, const float* lamb_p, bool nt, hipStream_t s)
{
    switch (err_dtype) {
    case OB_BF16: return ob::launch_chunk_sumsq<OB_BF16>(pd1, g, bf, err, clip, lamb_p, nt, s);
    case OB_F16: return ob::launch_chunk_sumsq<OB_F16>(pd1, g, bf, err, clip, lamb_p, nt, s);
    default: return ob::launch_chunk_sumsq<OB_F32>(pd1, g, bf, err, clip, lamb_p, nt, s);
    }
}

hipError_t compress_by_format(ob_dtype err_dtype, const ob::PlanDev& pd, const void* g, int bf, void* err,
                              float* m, const float* v, float* p, uint32_t* words, float* scales, int8_t* signs,
                              unsigned long long* nf, int ema, int lamb, const ob::CompressParams& cp,
                              hipStream_t s)
{
    switch (err_dtype) {
    case OB_BF16:
        return ob::launch_compress<OB_BF16>(pd, g, bf, err, m, v, p, words, scales, signs, nf, ema, lamb, cp, s);
    case OB_F16:
        return ob::launch_compress<OB_F16>(pd, g, bf, err, m, v, p, words, scales, signs, nf, ema, lamb, cp, s);
    default:
        return ob::launch_compress<OB_F32>(pd, g, bf, err, m, v, p, words, scales, signs, nf, ema, lamb, cp, s);
    }
}

// Pass-2 view of the plan.  With many partials per chunk, the chunk sums are formed first (one block
// per chunk) and the view's pass-1 table becomes the identity over them, so that each pass-2 block
// forms its scale from one partial instead of all of them.
ob_status pass2_view(ob_plan plan, int table, hipStream_t stream, ob::PlanDev* out, hipEvent_t* chain = nullptr)
{
    *out = plan->dev(table);
    if (plan->p1_max <= kFinalizeAt) return OB_OK;
    const ob::PlanDev pd1 = plan->dev(T_PASS1);
    const ob_status st = timed(
        plan, OB_KERNEL_SCALE, stream, [&] { return ob::launch_chunk_sums(pd1, plan->d_chunk_sums, stream); },
        chain);
    out->p1_first = plan->d_ident;
    out->partials = plan->d_chunk_sums;
    return st;
}

ob::CompressParams compress_params(const ob_hparams* hp)
{
    ob::CompressParams cp;
    cp.lr = hp->lr;
    cp.beta1 = hp->beta1;
    cp.one_m_beta1 = 1.0 - static_cast<double>(hp->beta1);
    cp.eps = hp->eps;
    cp.clip = hp->clip > 0.0f ? hp->clip : 0.0f;
    cp.ef_beta = hp->ef_beta;
    cp.one_m_ef_beta = 1.0 - static_cast<double>(hp->ef_beta);
    cp.stochastic = hp->err_rounding == OB_ROUND_STOCHASTIC;
    cp.sr_seed = hp->sr_seed;
    cp.sr_step = static_cast<uint64_t>(hp->step);
    return cp;
}

// Validation and passes 1-2 of the compressed step.  lamb != 0: passes 1-2 of the 1-bit LAMB step
// (sums of p^2 and u^2 instead of the update); the caller then runs the trust ratio and the update.
ob_status compress_passes(ob_plan plan, const void* g, ob_dtype g_dtype, void* err, ob_dtype err_dtype,
                          float* m, const float* v, float* p, uint32_t* words_out, float* scales_out,
                          int8_t* signs_out, uint64_t* nonfinite_out, const ob_hparams* hp, int lamb,
                          hipStream_t stream)
{
    if (!plan || !hp) return OB_ERR_ARG;
    if (!valid_dtype(g_dtype) || !valid_err_dtype(err_dtype)) return OB_ERR_DTYPE;
    if (plan->n == 0) return OB_OK;
    if (ob_status st = check_compress_args(g, g_dtype, err, err_dtype, m, v, p, words_out, scales_out, signs_out,
                                           nonfinite_out, hp))
        return st;
    if (lamb && (!lamb_fits(plan, T_PASS1, true, false) || !lamb_fits(plan, T_COMPRESS, false, true)))
        return OB_ERR_ARG;
    const ob::CompressParams cp = compress_params(hp);

    DeviceGuard guard(plan->device);
    if (!guard.ok) return OB_ERR_HIP;
    const ob::PlanDev pd1 = plan->dev(T_PASS1);
    ob::PlanDev pd;
    const int bf = g_dtype == OB_BF16;
    const int ema = hp->ef_mode == OB_EF_EMA;
    auto nf = reinterpret_cast<unsigned long long*>(nonfinite_out);
    const float* lamb_p = lamb ? p : nullptr;
    ob_status st = OB_OK;
    hipEvent_t chain = nullptr;
    const std::vector<ob::ChunkGroup>& groups = step_groups(plan, g_dtype, err_dtype, lamb);
    const bool whole = groups.size() == 1;   // one pass 1 over everything: nontemporal loads
    for (const ob::ChunkGroup& gr : groups) {
        st = timed(
            plan, OB_KERNEL_CHUNK_SUMSQ, stream,
            [&] {
                return sumsq_by_format(err_dtype, group_view(pd1, gr.i1, gr.n1), g, bf, err, cp.clip, lamb_p, whole,
                                       stream);
            },
            &chain);
        if (st != OB_OK) return st;
        if ((st = pass2_view(plan, T_COMPRESS, stream, &pd, &chain)) != OB_OK) return st;
        st = timed(
            plan, OB_KERNEL_COMPRESS, stream,
            [&] {
                return compress_by_format(err_dtype, group_view(pd, gr.i2, gr.n2), g, bf, err, m, v, p, words_out,
                                          scales_out, signs_out, nf, ema, lamb, cp, stream);
            },
            &chain);
        if (st != OB_OK) return st;
    }
    if (!plan->diag_err_sumsq) return st;
    const ob::PlanDev pdd = plan->dev(T_COMPRESS);   // the pass-1 table the error sums were written by
    return timed(plan, OB_KERNEL_DIAG, stream, [&] {
        return ob::launch_diag_reduce(pdd, plan->diag_err_sumsq, plan->diag_plus, stream);
    });
}

ob::LambParams lamb_params(const ob_hparams* hp, double bc1, double bc2)
{
    ob::LambParams lp;
    lp.lr = hp->lr;
    lp.eps = hp->eps;
    lp.bc1 = bc1;
    lp.bc2 = bc2;
    return lp;
}

// Trust ratios of every layer from the per-block sums (tables w_table / u_table), then the update on
// the dense block table.
ob_status lamb_finish(ob_plan plan, int w_table, int u_table, const float* m, const float* v, float* p,
                      float* ratios_out, int bias_correction, const ob::LambParams& lp, hipStream_t stream)
{
    ob::PlanDev pr = plan->dev(T_DENSE);
    pr.w_first = plan->t[w_table].d_first;
    pr.u_first = plan->t[u_table].d_first;
    ob_status st = timed(plan, OB_KERNEL_TRUST_RATIO, stream,
                         [&] { return ob::launch_trust_ratio(pr, ratios_out, stream); });
    if (st != OB_OK) return st;
    const ob::PlanDev pa = plan->dev(T_DENSE);
    return timed(plan, OB_KERNEL_LAMB_APPLY, stream, [&] {
        return ob::launch_lamb_apply(pa, m, v, p, ratios_out, bias_correction, lp, stream);
    });
}

}  // namespace

extern "C" {

ob_status ob_adam_compress_step(ob_plan plan, const void* g, ob_dtype g_dtype, void* err, ob_dtype err_dtype,
                                float* m, const float* v, float* p, uint32_t* words_out, float* scales_out,
                                int8_t* signs_out, uint64_t* nonfinite_out, const ob_hparams* hp,
                                hipStream_t stream)
try {
    return compress_passes(plan, g, g_dtype, err, err_dtype, m, v, p, words_out, scales_out, signs_out,
                           nonfinite_out, hp, 0, stream);
} catch (...) {
    return OB_ERR_OOM;  // host allocation failures are the only exceptions here
}

ob_status ob_adam_worker_compress(ob_plan plan, const void* g, ob_dtype g_dtype, void* err, ob_dtype err_dtype,
                                  uint32_t* words_out, float* scales_out, int8_t* signs_out,
                                  uint64_t* nonfinite_out, const ob_hparams* hp, hipStream_t stream)
try {
    if (!plan || !hp) return OB_ERR_ARG;
    if (!valid_dtype(g_dtype) || !valid_err_dtype(err_dtype)) return OB_ERR_DTYPE;
    if (plan->n == 0) return OB_OK;
    if (ob_status st = check_grad(g, g_dtype)) return st;
    if (!err || !words_out || !scales_out) return OB_ERR_ARG;
    if (!aligned(err, err_dtype == OB_F32 ? 16 : 8)) return OB_ERR_ALIGN;
    if (!aligned(words_out, 4) || !aligned(scales_out, 4)) return OB_ERR_ALIGN;
    if (signs_out && !aligned(signs_out, 4)) return OB_ERR_ALIGN;
    if (nonfinite_out && !aligned(nonfinite_out, 8)) return OB_ERR_ALIGN;
    if (hp->ef_mode != OB_EF_PLAIN && hp->ef_mode != OB_EF_EMA) return OB_ERR_ARG;
    if (hp->err_rounding != OB_ROUND_NEAREST && hp->err_rounding != OB_ROUND_STOCHASTIC) return OB_ERR_ARG;
    if (hp->err_rounding == OB_ROUND_STOCHASTIC && err_dtype == OB_F32) return OB_ERR_ARG;
    const ob::CompressParams cp = compress_params(hp);
    DeviceGuard guard(plan->device);
    if (!guard.ok) return OB_ERR_HIP;
    const ob::PlanDev pd1 = plan->dev(T_PASS1);
    const int bf = g_dtype == OB_BF16;
    const int ema = hp->ef_mode == OB_EF_EMA;
    auto nf = reinterpret_cast<unsigned long long*>(nonfinite_out);
    ob_status st = OB_OK;
    hipEvent_t chain = nullptr;
    const std::vector<ob::ChunkGroup>& groups = step_groups(plan, g_dtype, err_dtype, 0);
    const bool whole = groups.size() == 1;   // one pass 1 over everything: nontemporal loads
    for (const ob::ChunkGroup& gr : groups) {
        st = timed(
            plan, OB_KERNEL_CHUNK_SUMSQ, stream,
            [&] {
                return sumsq_by_format(err_dtype, group_view(pd1, gr.i1, gr.n1), g, bf, err, cp.clip, nullptr, whole,
                                       stream);
            },
            &chain);
        if (st != OB_OK) return st;
        ob::PlanDev pd;
        if ((st = pass2_view(plan, T_COMPRESS, stream, &pd, &chain)) != OB_OK) return st;
        const ob::PlanDev pg = group_view(pd, gr.i2, gr.n2);
        st = timed(plan, OB_KERNEL_WORKER_COMPRESS, stream, [&] {
            switch (err_dtype) {
            case OB_BF16:
                return ob::launch_worker_compress<OB_BF16>(pg, g, bf, err, words_out, scales_out, signs_out, nf, ema,
                                                           cp, stream);
            case OB_F16:
                return ob::launch_worker_compress<OB_F16>(pg, g, bf, err, words_out, scales_out, signs_out, nf, ema,
                                                          cp, stream);
            default:
                return ob::launch_worker_compress<OB_F32>(pg, g, bf, err, words_out, scales_out, signs_out, nf, ema,
                                                          cp, stream);
            }
        }, &chain);
        if (st != OB_OK) return st;
    }
    return st;
} catch (...) {
    return OB_ERR_OOM;  // host allocation failures are the only exceptions here
}

ob_status ob_adam_worker_update(ob_plan plan, const uint32_t* words, const float* scales, float* m,
                                const float* v, float* p, const ob_hparams* hp, hipStream_t stream)
try {
    if (!plan || !hp) return OB_ERR_ARG;
    if (plan->n == 0) return OB_OK;
    if (!words || !scales || !m || !v || !p) return OB_ERR_ARG;
    if (!aligned(words, 4) || !aligned(scales, 4)) return OB_ERR_ALIGN;
    if (!aligned(m, 16) || !aligned(v, 16) || !aligned(p, 16)) return OB_ERR_ALIGN;
    const ob::CompressParams cp = compress_params(hp);
    DeviceGuard guard(plan->device);
    if (!guard.ok) return OB_ERR_HIP;
    const ob::PlanDev pd = plan->dev(T_COMPRESS);
    return timed(plan, OB_KERNEL_WORKER_UPDATE, stream,
                 [&] { return ob::launch_worker_update(pd, words, scales, m, v, p, 0, cp, stream); });
} catch (...) {
    return OB_ERR_OOM;  // host allocation failures are the only exceptions here
}

ob_status ob_lamb_worker_update(ob_plan plan, const uint32_t* words, const float* scales, float* m,
                                const float* v, float* p, float* ratios_out, const ob_hparams* hp,
                                hipStream_t stream)
try {
    if (!plan || !hp) return OB_ERR_ARG;
    if (plan->n == 0) return OB_OK;
    if (!words || !scales || !m || !v || !p || !ratios_out) return OB_ERR_ARG;
    if (!aligned(words, 4) || !aligned(scales, 4) || !aligned(ratios_out, 4)) return OB_ERR_ALIGN;
    if (!aligned(m, 16) || !aligned(v, 16) || !aligned(p, 16)) return OB_ERR_ALIGN;
    if (!lamb_fits(plan, T_COMPRESS, true, true)) return OB_ERR_ARG;
    const ob::CompressParams cp = compress_params(hp);
    DeviceGuard guard(plan->device);
    if (!guard.ok) return OB_ERR_HIP;
    const ob::PlanDev pd = plan->dev(T_COMPRESS);
    ob_status st = timed(plan, OB_KERNEL_WORKER_UPDATE, stream,
                         [&] { return ob::launch_worker_update(pd, words, scales, m, v, p, 1, cp, stream); });
    if (st != OB_OK) return st;
    return lamb_finish(plan, T_COMPRESS, T_COMPRESS, m, v, p, ratios_out, 0, lamb_params(hp, 1.0, 1.0), stream);
} catch (...) {
    return OB_ERR_OOM;  // host allocation failures are the only exceptions here
}

ob_status ob_lamb_compress_step(ob_plan plan, const void* g, ob_dtype g_dtype, void* err, ob_dtype err_dtype,
                                float* m, const float* v, float* p, uint32_t* words_out, float* scales_out,
                                float* ratios_out, int8_t* signs_out, uint64_t* nonfinite_out,
                                const ob_hparams* hp, hipStream_t stream)
try {
    if (!plan || !hp) return OB_ERR_ARG;
    if (plan->n > 0 && (!ratios_out || !aligned(ratios_out, 4))) return ratios_out ? OB_ERR_ALIGN : OB_ERR_ARG;
    ob_status st = compress_passes(plan, g, g_dtype, err, err_dtype, m, v, p, words_out, scales_out, signs_out,
                                   nonfinite_out, hp, 1, stream);
    if (st != OB_OK || plan->n == 0) return st;
    DeviceGuard guard(plan->device);
    if (!guard.ok) return OB_ERR_HIP;
    return lamb_finish(plan, T_PASS1, T_COMPRESS, m, v, p, ratios_out, 0, lamb_params(hp, 1.0, 1.0), stream);
} catch (...) {
    return OB_ERR_OOM;  // host allocation failures are the only exceptions here
}

ob_status ob_lamb_warmup_step(ob_plan plan, const void* g, ob_dtype g_dtype, float* m, float* v, float* p,
                              float* ratios_out, const ob_hparams* hp, hipStream_t stream)
try {
    if (!plan || !hp) return OB_ERR_ARG;
    if (!valid_dtype(g_dtype)) return OB_ERR_DTYPE;
    if (plan->n == 0) return OB_OK;
    if (ob_status st = check_grad(g, g_dtype)) return st;
    if (!m || !v || !p || !ratios_out) return OB_ERR_ARG;
    if (!aligned(m, 16) || !aligned(v, 16) || !aligned(p, 16) || !aligned(ratios_out, 4)) return OB_ERR_ALIGN;
    if (hp->bias_correction && hp->step < 1) return OB_ERR_ARG;
    if (!lamb_fits(plan, T_DENSE, true, true)) return OB_ERR_ARG;
    const ob::DenseParams dp = dense_params(hp);
    DeviceGuard guard(plan->device);
    if (!guard.ok) return OB_ERR_HIP;
    const ob::PlanDev pd = plan->dev(T_DENSE);
    const int bf = g_dtype == OB_BF16;
    ob_status st = timed(plan, OB_KERNEL_DENSE, stream,
                         [&] { return ob::launch_dense(pd, g, bf, m, v, p, 1, dp, stream); });
    if (st != OB_OK) return st;
    return lamb_finish(plan, T_DENSE, T_DENSE, m, v, p, ratios_out, dp.bias_correction,
                       lamb_params(hp, dp.bc1, dp.bc2), stream);
} catch (...) {
    return OB_ERR_OOM;  // host allocation failures are the only exceptions here
}

ob_status ob_server_reduce(ob_plan plan, int32_t W, const uint32_t* worker_words, const float* worker_scales,
                           float* server_err, uint32_t* words_out, float* scales_out, hipStream_t stream)
try {
    if (!plan) return OB_ERR_ARG;
    if (W < 1 || W > 1024) return OB_ERR_ARG;
    if (plan->n == 0) return OB_OK;
    if (!worker_words || !worker_scales || !server_err || !words_out || !scales_out) return OB_ERR_ARG;
    if (!aligned(worker_words, 4) || !aligned(worker_scales, 4) || !aligned(server_err, 16) ||
        !aligned(words_out, 4) || !aligned(scales_out, 4))
        return OB_ERR_ALIGN;
    DeviceGuard guard(plan->device);
    if (!guard.ok) return OB_ERR_HIP;
    const ob::PlanDev pd1 = plan->dev(T_PASS1);
    ob_status st = timed(plan, OB_KERNEL_SERVER_SUMSQ, stream, [&] {
        return ob::launch_server_sumsq(pd1, W, worker_words, worker_scales, server_err, plan->off128, stream);
    });
    if (st != OB_OK) return st;
    ob::PlanDev pd;
    if ((st = pass2_view(plan, T_SERVER, stream, &pd)) != OB_OK) return st;
    return timed(plan, OB_KERNEL_SERVER_APPLY, stream, [&] {
        return ob::launch_server_apply(pd, W, worker_words, worker_scales, server_err, words_out, scales_out,
                                       stream);
    });
} catch (...) {
    return OB_ERR_OOM;  // host allocation failures are the only exceptions here
}

ob_status ob_pack(const void* x, ob_dtype x_dtype, int64_t n, uint32_t* words_out, hipStream_t stream)
try {
    if (!valid_dtype(x_dtype)) return OB_ERR_DTYPE;
    if (n < 0) return OB_ERR_ARG;
    if (n == 0) return OB_OK;
    if (!x || !words_out) return OB_ERR_ARG;
    if (n > int64_t(INT32_MAX) * ob::kPlainItem) return OB_ERR_ARG;
    if (!aligned(x, x_dtype == OB_BF16 ? 8 : 16) || !aligned(words_out, 4)) return OB_ERR_ALIGN;
    (void)hipGetLastError();
    return ob::launch_pack(x, x_dtype == OB_BF16, n, words_out, stream) == hipSuccess ? OB_OK : OB_ERR_HIP;
} catch (...) {
    return OB_ERR_OOM;  // host allocation failures are the only exceptions here
}

ob_status ob_unpack(ob_plan plan, const uint32_t* words, int64_t n, const float* scales, float* out,
                    hipStream_t stream)
try {
    if (n < 0) return OB_ERR_ARG;
    if (scales && !plan) return OB_ERR_ARG;
    if (plan && plan->n != n) return OB_ERR_ARG;
    if (n == 0) return OB_OK;
    if (!words || !out) return OB_ERR_ARG;
    if (!aligned(words, 4) || !aligned(out, 16) || (scales && !aligned(scales, 4))) return OB_ERR_ALIGN;
    if (plan && scales) {
        DeviceGuard guard(plan->device);
        if (!guard.ok) return OB_ERR_HIP;
        const ob::PlanDev pd = plan->dev(T_SERVER);
        return timed(plan, OB_KERNEL_UNPACK, stream,
                     [&] { return ob::launch_unpack(&pd, words, n, scales, out, stream); });
    }
    if (n > int64_t(INT32_MAX) * ob::kPlainItem) return OB_ERR_ARG;
    (void)hipGetLastError();
    return ob::launch_unpack(nullptr, words, n, nullptr, out, stream) == hipSuccess ? OB_OK : OB_ERR_HIP;
} catch (...) {
    return OB_ERR_OOM;  // host allocation failures are the only exceptions here
}

ob_status ob_adam_compress_step_noalloc(int64_t n, int64_t chunk_size, const void* g, ob_dtype g_dtype,
                                        void* err, ob_dtype err_dtype, float* m, const float* v, float* p,
                                        uint32_t* words_out, float* scales_out, int8_t* signs_out,
                                        uint64_t* nonfinite_out, const ob_hparams* hp, hipStream_t stream)
try {
    // everything up to the size check is host arithmetic: a rejected call makes no HIP call
    if (!hp) return OB_ERR_ARG;
    if (!valid_dtype(g_dtype) || !valid_err_dtype(err_dtype)) return OB_ERR_DTYPE;
    if (n < 0 || chunk_size <= 0) return OB_ERR_ARG;
    if (n == 0) return OB_OK;
    if (ob_status st = check_compress_args(g, g_dtype, err, err_dtype, m, v, p, words_out, scales_out, signs_out,
                                           nonfinite_out, hp))
        return st;
    const int64_t K = (n + chunk_size - 1) / chunk_size;
    if (K > 1 && chunk_size % 64 != 0) return OB_ERR_ALIGN;
    if (K > INT32_MAX - 1) return OB_ERR_SIZE;

    // the block tables ob_plan_create would build for these uniform chunks (same block sizes)
    const int64_t be1 = choose_block_elems(n, T_PASS1), be2 = choose_block_elems(n, T_COMPRESS);
    const int64_t last = n - (K - 1) * chunk_size;
    auto blocks = [](int64_t len, int64_t be) { return (len + be - 1) / be; };
    const int64_t nbf1 = K > 1 ? blocks(chunk_size, be1) : 0, nbf2 = K > 1 ? blocks(chunk_size, be2) : 0;
    const int64_t n1 = (K - 1) * nbf1 + blocks(last, be1), n2 = (K - 1) * nbf2 + blocks(last, be2);
    const bool finalize = std::max(nbf1, blocks(last, be1)) > kFinalizeAt;

    // layout of the static buffer: every region starts on a 256-byte boundary
    int64_t used = 0;
    auto region = [&](int64_t bytes) {
        const int64_t at = used;
        used += (bytes + 255) / 256 * 256;
        return at;
    };
    const int64_t o_items1 = region(n1 * int64_t(sizeof(ob::Item))), o_first1 = region((K + 1) * 4);
    const int64_t o_items2 = region(n2 * int64_t(sizeof(ob::Item))), o_first2 = region((K + 1) * 4);
    const int64_t o_off = region((K + 1) * 8), o_part = region(n1 * 8);
    const int64_t o_sums = finalize ? region(K * 8) : 0, o_ident = finalize ? region((K + 1) * 4) : 0;
    if (used > ob::kNoallocScratchBytes || n1 > INT32_MAX || n2 > INT32_MAX) return OB_ERR_SIZE;

    int device = 0;
    if (hipGetDevice(&device) != hipSuccess) return OB_ERR_HIP;
    unsigned char* base = static_cast<unsigned char*>(ob::noalloc_scratch(device));
    if (!base) return OB_ERR_HIP;

    ob::UniformTables t;
    t.items1 = reinterpret_cast<ob::Item*>(base + o_items1);
    t.first1 = reinterpret_cast<int32_t*>(base + o_first1);
    t.items2 = reinterpret_cast<ob::Item*>(base + o_items2);
    t.first2 = reinterpret_cast<int32_t*>(base + o_first2);
    t.off = reinterpret_cast<int64_t*>(base + o_off);
    t.ident = finalize ? reinterpret_cast<int32_t*>(base + o_ident) : nullptr;
    t.n = n;
    t.chunk = chunk_size;
    t.be1 = be1;
    t.be2 = be2;
    t.n1 = n1;
    t.n2 = n2;
    t.K = static_cast<int32_t>(K);
    t.nbf1 = static_cast<int32_t>(nbf1);
    t.nbf2 = static_cast<int32_t>(nbf2);

    // the views a plan's dev() would give: pass 1 over items1, the fused pass over items2
    ob::PlanDev pd1 = {};
    pd1.items = t.items1;
    pd1.chunk_first = t.first1;
    pd1.p1_first = t.first1;
    pd1.chunk_off = t.off;
    pd1.partials = reinterpret_cast<double*>(base + o_part);
    pd1.n = n;
    pd1.n_items = n1;
    pd1.K = t.K;
    ob::PlanDev pd2 = pd1;
    pd2.items = t.items2;
    pd2.chunk_first = t.first2;
    pd2.n_items = n2;

    const ob::CompressParams cp = compress_params(hp);
    const int bf = g_dtype == OB_BF16;
    const int ema = hp->ef_mode == OB_EF_EMA;
    auto nf = reinterpret_cast<unsigned long long*>(nonfinite_out);
    (void)hipGetLastError();
    if (ob::launch_uniform_tables(t, stream) != hipSuccess) return OB_ERR_HIP;
    if (finalize) {   // chunks too large to share the cache: whole-buffer passes, with per-chunk sums
        if (sumsq_by_format(err_dtype, pd1, g, bf, err, cp.clip, nullptr, true, stream) != hipSuccess)
            return OB_ERR_HIP;
        double* sums = reinterpret_cast<double*>(base + o_sums);
        if (ob::launch_chunk_sums(pd1, sums, stream) != hipSuccess) return OB_ERR_HIP;
        pd2.p1_first = t.ident;
        pd2.partials = sums;
        return compress_by_format(err_dtype, pd2, g, bf, err, m, v, p, words_out, scales_out, signs_out, nf, ema,
                                  0, cp, stream) == hipSuccess
                   ? OB_OK
                   : OB_ERR_HIP;
    }
    // chunk groups of q chunks (the plan's greedy grouping, for equal chunks; the last group takes the rest)
    const int64_t budget = group_budget();
    const int64_t width = (g_dtype == OB_BF16 ? 2 : 4) + (err_dtype == OB_F32 ? 4 : 2);
    const int64_t max_elems = budget > 0 ? std::max<int64_t>(1, budget / width) : 0;
    const int64_t q = max_elems > 0 ? std::max<int64_t>(1, max_elems / chunk_size) : K;
    const bool whole = q >= K;   // one group: nontemporal pass-1 loads
    for (int64_t c0 = 0; c0 < K; c0 += q) {
        const ob::ChunkGroup gr = ob::uniform_chunk_group(c0, q, K, nbf1, n1, nbf2, n2);
        if (sumsq_by_format(err_dtype, group_view(pd1, gr.i1, gr.n1), g, bf, err, cp.clip, nullptr, whole,
                            stream) != hipSuccess)
            return OB_ERR_HIP;
        if (compress_by_format(err_dtype, group_view(pd2, gr.i2, gr.n2), g, bf, err, m, v, p, words_out, scales_out,
                               signs_out, nf, ema, 0, cp, stream) != hipSuccess)
            return OB_ERR_HIP;
    }
    return OB_OK;
} catch (...) {
    return OB_ERR_OOM;  // host allocation failures are the only exceptions here
}

ob_status ob_plan_set_diagnostics(ob_plan plan, double* err_sumsq_out, uint64_t* plus_count_out)
try {
    if (!plan) return OB_ERR_ARG;
    if ((err_sumsq_out == nullptr) != (plus_count_out == nullptr)) return OB_ERR_ARG;
    if (err_sumsq_out && (!aligned(err_sumsq_out, 8) || !aligned(plus_count_out, 8))) return OB_ERR_ALIGN;
    if (err_sumsq_out && plan->n > 0 && !plan->d_partials_e) {
        DeviceGuard guard(plan->device);
        if (!guard.ok) return OB_ERR_HIP;
        hipError_t e = hipMalloc(&plan->d_partials_e, plan->t[T_PASS1].n_items * sizeof(double));
        if (e == hipSuccess)
            e = hipMalloc(&plan->d_partials_b, plan->t[T_COMPRESS].n_items * sizeof(uint32_t));
        if (e != hipSuccess) {
            if (plan->d_partials_e) (void)hipFree(plan->d_partials_e);
            plan->d_partials_e = nullptr;
            plan->d_partials_b = nullptr;
            return e == hipErrorOutOfMemory ? OB_ERR_OOM : OB_ERR_HIP;
        }
    }
    plan->diag_err_sumsq = err_sumsq_out;
    plan->diag_plus = reinterpret_cast<unsigned long long*>(plus_count_out);
    return OB_OK;
} catch (...) {
    return OB_ERR_OOM;  // host allocation failures are the only exceptions here
}

ob_status ob_plan_set_timing(ob_plan plan, int32_t enable)
try {
    if (!plan) return OB_ERR_ARG;
    DeviceGuard guard(plan->device);
    ob_status st = drain_timing(plan);
    plan->timing = enable != 0;
    for (int k = 0; k < OB_KERNEL_COUNT; ++k) {
        plan->total_ms[k] = 0.0;
        plan->launches[k] = 0;
    }
    return st;
} catch (...) {
    return OB_ERR_OOM;  // host allocation failures are the only exceptions here
}

ob_status ob_plan_read_timing(ob_plan plan, int32_t kernel, double* total_ms, int64_t* launches)
try {
    if (!plan || kernel < 0 || kernel >= OB_KERNEL_COUNT || !total_ms || !launches) return OB_ERR_ARG;
    DeviceGuard guard(plan->device);
    const ob_status st = drain_timing(plan);
    *total_ms = plan->total_ms[kernel];
    *launches = plan->launches[kernel];
    return st;
} catch (...) {
    return OB_ERR_OOM;  // host allocation failures are the only exceptions here
}

}  // extern "C"
