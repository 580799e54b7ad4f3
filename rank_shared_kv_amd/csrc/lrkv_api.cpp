// C ABI of the LRKV decode library: argument checks, split planning and
// kernel launches.  Everything here is host code; no HIP call is made before
// a call's arguments have been checked, and nothing runs at load time.
#include "lrkv.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <mutex>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "lrkv_device.hpp"
#include "lrkv_internal.hpp"
#include "lrkv_step.hpp"

namespace {

thread_local char g_last_error[512] = "";

lrkv_status fail(lrkv_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return st;
}

lrkv_status ok() {
    g_last_error[0] = '\0';
    return LRKV_OK;
}

lrkv_status hip_fail(hipError_t e, const char* what) {
    return fail(LRKV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool dims_valid(const lrkv_dims* d) {
    return d && d->batch >= 1 && d->batch <= 65535 && d->H >= 1 && d->H <= 1024 && d->d_h >= 1 && d->d_h <= 4096 &&
           d->r >= 0 && d->r <= 4096 && d->L_cap >= 1 && d->L_cap <= (1 << 28) &&
           (d->dtype == LRKV_F32 || d->dtype == LRKV_BF16);
}

lrkv_status check_dims(const lrkv_dims* d) {
    if (!d) return fail(LRKV_ERR_INVALID_ARG, "dims is NULL");
    if (!dims_valid(d))
        return fail(LRKV_ERR_INVALID_ARG, "invalid dims (batch=%d H=%d d_h=%d r=%d L_cap=%d dtype=%d)", d->batch, d->H,
                    d->d_h, d->r, d->L_cap, d->dtype);
    return LRKV_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

lrkv_status need_ptr(const void* p, const char* name) {
    if (!p) return fail(LRKV_ERR_INVALID_ARG, "%s is NULL", name);
    if (!aligned16(p)) return fail(LRKV_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
    return LRKV_OK;
}

#define LRKV_TRY(expr)                  \
    do {                                \
        lrkv_status _s = (expr);        \
        if (_s != LRKV_OK) return _s;   \
    } while (0)

// Device scratch of lrkv_decode_noalloc: the split records of one decode, in a static device array instead of
// a caller's workspace.  Each GPU the library runs on holds its own copy from the first call on it until the
// process ends.  Host code never uses the array's name as an address: its device address comes from
// hipGetSymbolAddress, once per device with that device current, and is kept in scratch_ptr[].
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on device `dev` (NULL with *err set on failure).
void* scratch_on(int dev, hipError_t* err) {
    *err = hipSuccess;
    if (dev < 0 || dev >= kMaxDevices) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev]) return g_scratch_ptr[dev];
    int cur = -1;
    if ((*err = hipGetDevice(&cur)) != hipSuccess) return nullptr;
    if (cur != dev && (*err = hipSetDevice(dev)) != hipSuccess) return nullptr;
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != dev) {
        const hipError_t e2 = hipSetDevice(cur);
        if (e == hipSuccess && e2 != hipSuccess) {
            *err = e2;
            return nullptr;
        }
    }
    if (e != hipSuccess || !ptr) {
        *err = e != hipSuccess ? e : hipErrorInvalidSymbol;
        return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
    return ptr;
}

int env_int(const char* name, int dflt) {
    const char* v = getenv(name);
    if (!v || !*v) return dflt;
    char* end = nullptr;
    long x = strtol(v, &end, 10);
    return (end && *end == '\0' && x > 0 && x < (1L << 30)) ? (int)x : dflt;
}

// Split planning.  Pure arithmetic on (dims, max_len) so that workspace sizes are known on the host without a
// device.  A plan is (G workgroups for the whole batch, granule g in rows).  On the device the G workgroups are
// dealt to the sequences by their lengths, at least one each (lrkv_device.hpp: the fewest splits under a common
// cap on a row lane's blocks when that cap is long, else in proportion to the lengths); split s of sequence b
// takes the g-row tiles s, s + S_b, ... of the sequence and writes partial record W_b + s.  G aims at one
// resident round of workgroups (MI355X has 256 CUs; the matrix-core kernels hold `occupancy` workgroups per
// CU), never fewer than one per sequence nor more than one per tile of every sequence.  The plan does not depend
// on r within a kernel, so problems differing only in rank reduce in the same order.
// Tuning overrides (read at every call, so they must not change between a workspace query and the decode that
// uses it): LRKV_OCCUPANCY (1 or 2 waves per SIMD; defaults: 2 for the fp32 matrix-core kernel, 2 for the bf16
// one at batch >= 32 and 1 below), LRKV_TARGET_WGS (G before clamping), LRKV_SPLITS (G = splits x batch),
// LRKV_FORCE_GENERAL (1: the general kernel for the plain decode).
constexpr long kMaxExtraSplits = 8192;  // G - batch: bounds the merge kernel's LDS

// Which decode the plan is for.  The normalised variant's bf16 matrix-core kernel is built for one wave per
// SIMD; neither it nor the paged cache has an fp32 matrix-core kernel (the general kernel serves them).  Their
// G never exceeds the plain plan's, so the plain workspace size serves them, and a paged decode of a bf16
// matrix-core shape uses exactly the plain plan.  The rotary variant has kernels of its own (one
// eight-wave workgroup per CU for the bf16 one) and its own workspace query.  Query sets (multi-token decode with
// several tokens per workgroup) run the bf16 matrix-core kernel at one wave per SIMD.
enum class PlanVariant { kPlain, kNormed, kPaged, kRope, kQuerySets };

bool plan_split(const lrkv_dims& d, int max_len, lrkv::SplitPlan* out, PlanVariant variant = PlanVariant::kPlain) {
    using namespace lrkv;
    SplitPlan p{};
    if (variant != PlanVariant::kPlain) {
        SplitPlan plain;
        if (!plan_split(d, max_len, &plain)) return false;
        if (variant == PlanVariant::kPaged && plain.path != SplitPath::kMfmaF32) {
            *out = plain;
            return true;
        }
        if (variant == PlanVariant::kRope && rope_mfma_path_supports(d.H, d.d_h, d.r, d.dtype)) {
            p.path = SplitPath::kRopeMfma;
            p.chunk = rope_mfma_rows_per_tile();
        } else if (variant != PlanVariant::kRope && mfma_path_supports(d.H, d.d_h, d.r, d.dtype, d.L_cap) &&
                   mfma_all_variants(d.H, d.d_h, d.r)) {
            p.path = SplitPath::kMfmaBf16;
            p.chunk = mfma_rows_per_tile(d.H);
        } else if (variant == PlanVariant::kRope ? general_lds_bytes(d.H, d.d_h, d.r, true) <= 160 * 1024 &&
                                                       general_path_supports(d.H, d.d_h, d.r)
                                                 : general_path_supports(d.H, d.d_h, d.r)) {
            p.path = SplitPath::kGeneral;
            p.chunk = general_rows_per_tile();
        } else {
            return false;
        }
        p.occupancy = 1;
        const long tiles_per_seq = max_len > 0 ? (max_len + p.chunk - 1) / p.chunk : 0;
        // one resident round of workgroups; capped by the plain plan except for the rotary variant
        long G = p.path == SplitPath::kGeneral ? 1024 : p.path == SplitPath::kRopeMfma ? rope_mfma_workgroups() : 256;
        if (variant != PlanVariant::kRope) G = std::min<long>(plain.num_splits, G);
        G = std::min<long>(G, (long)d.batch + kMaxExtraSplits);
        G = std::min<long>(G, (long)d.batch * tiles_per_seq);
        p.num_splits = max_len > 0 ? (int)std::max<long>(G, d.batch) : 0;
        if ((long long)p.num_splits * d.H * lrkv::partial_record_floats(d.d_h, d.r) >= (1LL << 31)) return false;
        *out = p;
        return true;
    }
    // LRKV_FORCE_GENERAL=1 runs the general kernel wherever it applies (comparisons of problems that would
    // otherwise take different kernels, e.g. fp32 rank 0 against fp32 rank r with zero latents)
    const bool force_general = env_int("LRKV_FORCE_GENERAL", 0) == 1 && general_path_supports(d.H, d.d_h, d.r);
    if (force_general) {
        p.path = SplitPath::kGeneral;
        p.occupancy = 1;
    } else if (mfma_path_supports(d.H, d.d_h, d.r, d.dtype, d.L_cap)) {
        p.path = SplitPath::kMfmaBf16;
        // two waves per SIMD pay off for large batches (many sequences, splits of few blocks each: the
        // 64-sequence ragged batch runs 4% faster) and cost 1-3% for a few long sequences; the choice
        // depends on the batch only, never on r, so problems differing only in rank share a plan
        p.occupancy = env_int("LRKV_OCCUPANCY", d.batch >= 32 ? 2 : 1) == 2 ? 2 : 1;
    } else if (mfma_f32_path_supports(d.H, d.d_h, d.r, d.dtype, d.L_cap)) {
        p.path = SplitPath::kMfmaF32;
        p.occupancy = env_int("LRKV_OCCUPANCY", 2) == 1 ? 1 : 2;  // two waves per SIMD hide its MFMA chains
    } else if (general_path_supports(d.H, d.d_h, d.r)) {
        p.path = SplitPath::kGeneral;
        p.occupancy = 1;
    } else {
        return false;
    }
    const bool mfma = p.path != SplitPath::kGeneral;
    p.chunk = (p.path == SplitPath::kMfmaBf16)  ? mfma_rows_per_tile(d.H)
              : (p.path == SplitPath::kMfmaF32) ? mfma_f32_rows_per_tile()
                                                 : general_rows_per_tile();
    if (max_len <= 0) {
        p.num_splits = 0;
        *out = p;
        return true;
    }
    const long tiles_per_seq = (max_len + p.chunk - 1) / p.chunk;
    long G = env_int("LRKV_TARGET_WGS", mfma ? 256 * p.occupancy : 1024);
    const int forced = env_int("LRKV_SPLITS", 0);
    if (forced > 0) G = (long)forced * d.batch;
    G = std::min<long>(G, (long)d.batch + kMaxExtraSplits);
    G = std::min<long>(G, (long)d.batch * tiles_per_seq);
    G = std::max<long>(G, d.batch);
    // the merge kernel addresses the workspace with 32-bit offsets
    if ((long long)G * d.H * lrkv::partial_record_floats(d.d_h, d.r) >= (1LL << 31)) return false;
    p.num_splits = (int)G;
    *out = p;
    return true;
}

size_t workspace_bytes(const lrkv_dims& d, const lrkv::SplitPlan& p) {
    return sizeof(float) * (size_t)p.num_splits * (size_t)d.H *
           (size_t)lrkv::partial_record_floats(d.d_h, d.r);
}

lrkv_status check_decode_common(const lrkv_dims* dims, int32_t max_len, lrkv::SplitPlan* plan,
                                PlanVariant variant = PlanVariant::kPlain) {
    LRKV_TRY(check_dims(dims));
    if (max_len < 0 || max_len > dims->L_cap)
        return fail(LRKV_ERR_INVALID_ARG, "max_len=%d outside [0, L_cap=%d]", max_len, dims->L_cap);
    if (!plan_split(*dims, max_len, plan, variant))
        return fail(LRKV_ERR_UNSUPPORTED, "no kernel for H=%d d_h=%d r=%d dtype=%d", dims->H, dims->d_h, dims->r,
                    dims->dtype);
    return LRKV_OK;
}

lrkv_status check_workspace(const lrkv_dims& d, const lrkv::SplitPlan& p, const void* ws, size_t ws_bytes) {
    const size_t need = workspace_bytes(d, p);
    if (need == 0) return LRKV_OK;
    if (!ws) return fail(LRKV_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", need);
    if (reinterpret_cast<uintptr_t>(ws) & 255u) return fail(LRKV_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
    if (ws_bytes < need) return fail(LRKV_ERR_WORKSPACE, "workspace has %zu bytes, need %zu", ws_bytes, need);
    return LRKV_OK;
}

struct PagedView {  // the paged layout of a cache handed to run_partial (block_table NULL: contiguous)
    const int32_t* block_table = nullptr;
    int page_shift = 0, max_pages = 0, n_pages = 0;
};

struct QuerySets {  // multi-token decode: virtual sequences of qw query tokens, qgroup per cached sequence
    int qgroup = 1, n_queries = 1, qw = 1;
};

lrkv_status run_partial(const lrkv_dims& d, const lrkv_cache& c, int max_len, const void* q, const float* p,
                        void* ws, const lrkv::SplitPlan& plan, hipStream_t stream, const void* rho = nullptr,
                        const PagedView& pv = PagedView(), const QuerySets& qs = QuerySets(),
                        const float* rope_cs = nullptr, const void* rope_bk = nullptr) {
    using namespace lrkv;
    if (plan.num_splits == 0) return LRKV_OK;
    DecodeArgs a{};
    a.batch = d.batch;
    a.H = d.H;
    a.d_h = d.d_h;
    a.r = d.r;
    a.L_cap = d.L_cap;
    a.dtype = d.dtype;
    a.max_len = max_len;
    a.chunk = plan.chunk;
    a.num_splits = plan.num_splits;
    a.qgroup = qs.qgroup;
    a.n_queries = qs.n_queries;
    a.qw = qs.qw;
    a.k_shared = c.k_shared;
    a.v_shared = c.v_shared;
    a.z_k = c.z_k;
    a.z_v = c.z_v;
    a.seq_lens = c.seq_lens;
    a.q = q;
    a.p = p;
    a.rho = rho;
    a.ws = (float*)ws;
    a.rope_cs = rope_cs;
    a.rope_bk = rope_bk;
    a.block_table = pv.block_table;
    a.page_shift = pv.page_shift;
    a.max_pages = pv.max_pages;
    a.n_pages = pv.n_pages;
    hipError_t e = (plan.path == SplitPath::kMfmaBf16)   ? launch_split_mfma(a, plan.occupancy, stream)
                   : (plan.path == SplitPath::kMfmaF32)  ? launch_split_mfma_f32(a, plan.occupancy, stream)
                   : (plan.path == SplitPath::kRopeMfma) ? launch_split_rope_mfma(a, stream)
                                                          : launch_split_general(a, stream);
    if (e != hipSuccess) return hip_fail(e, "split kernel launch");
    return LRKV_OK;
}

lrkv_status check_cache(const lrkv_dims& d, const lrkv_cache* c, bool need_latents) {
    if (!c) return fail(LRKV_ERR_INVALID_ARG, "cache is NULL");
    LRKV_TRY(need_ptr(c->k_shared, "cache.k_shared"));
    LRKV_TRY(need_ptr(c->v_shared, "cache.v_shared"));
    LRKV_TRY(need_ptr(c->seq_lens, "cache.seq_lens"));
    if (d.r > 0 && need_latents) {
        LRKV_TRY(need_ptr(c->z_k, "cache.z_k"));
        LRKV_TRY(need_ptr(c->z_v, "cache.z_v"));
    }
    return LRKV_OK;
}

}  // namespace

extern "C" {

const char* lrkv_status_str(lrkv_status s) {
    switch (s) {
        case LRKV_OK: return "LRKV_OK";
        case LRKV_ERR_INVALID_ARG: return "LRKV_ERR_INVALID_ARG";
        case LRKV_ERR_UNSUPPORTED: return "LRKV_ERR_UNSUPPORTED";
        case LRKV_ERR_WORKSPACE: return "LRKV_ERR_WORKSPACE";
        case LRKV_ERR_HIP: return "LRKV_ERR_HIP";
    }
    return "LRKV_UNKNOWN_STATUS";
}

const char* lrkv_last_error(void) { return g_last_error; }

uint64_t lrkv_cache_bytes(const lrkv_dims* dims, const int32_t* host_seq_lens) {
    if (!dims_valid(dims)) return 0;
    const uint64_t s = dims->dtype == LRKV_F32 ? 4 : 2;
    uint64_t rows = 0;
    for (int b = 0; b < dims->batch; ++b) {
        int64_t L = host_seq_lens ? host_seq_lens[b] : dims->L_cap;
        L = std::max<int64_t>(0, std::min<int64_t>(L, dims->L_cap));
        rows += (uint64_t)L;
    }
    return 2ull * s * rows * ((uint64_t)dims->d_h + (uint64_t)dims->H * (uint64_t)dims->r);
}

size_t lrkv_decode_workspace_bytes(const lrkv_dims* dims, int32_t max_len) {
    if (!dims_valid(dims) || max_len < 0 || max_len > dims->L_cap) return 0;
    lrkv::SplitPlan p;
    if (!plan_split(*dims, max_len, &p)) return 0;
    return workspace_bytes(*dims, p);
}

int32_t lrkv_decode_num_splits(const lrkv_dims* dims, int32_t max_len, int32_t* chunk_tokens) {
    if (!dims_valid(dims) || max_len <= 0 || max_len > dims->L_cap) return 0;
    lrkv::SplitPlan p;
    if (!plan_split(*dims, max_len, &p)) return 0;
    if (chunk_tokens) *chunk_tokens = p.chunk;
    return p.num_splits;
}

lrkv_status lrkv_decode_split_plan(const lrkv_dims* dims, int32_t max_len, const int32_t* seq_lens, int32_t append,
                                   int32_t* first_wg, int32_t* splits, void* stream) {
    lrkv::SplitPlan plan;
    LRKV_TRY(check_decode_common(dims, max_len, &plan));
    if (append != 0 && append != 1) return fail(LRKV_ERR_INVALID_ARG, "append=%d is neither 0 nor 1", append);
    LRKV_TRY(need_ptr(seq_lens, "seq_lens"));
    LRKV_TRY(need_ptr(first_wg, "first_wg"));
    LRKV_TRY(need_ptr(splits, "splits"));
    if (plan.num_splits == 0) return ok();  // max_len 0: no split workgroups, nothing written
    const hipError_t e = lrkv::launch_split_plan(dims->batch, max_len, append ? dims->L_cap : 0, plan.chunk,
                                                 plan.num_splits, seq_lens, first_wg, splits, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "split plan kernel launch");
    return ok();
}

lrkv_status lrkv_absorb_query(const lrkv_dims* dims, const void* q, const void* B_k, float* p, void* stream) {
    LRKV_TRY(check_dims(dims));
    if (dims->r == 0) return ok();
    LRKV_TRY(need_ptr(q, "q"));
    LRKV_TRY(need_ptr(B_k, "B_k"));
    LRKV_TRY(need_ptr(p, "p"));
    hipError_t e = lrkv::launch_absorb(dims->batch, dims->H, dims->d_h, dims->r, dims->dtype, q, B_k, p,
                                       (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "absorb kernel launch");
    return ok();
}

lrkv_status lrkv_cache_append(const lrkv_dims* dims, const lrkv_cache* cache, const void* k_new, const void* v_new,
                              const void* zk_new, const void* zv_new, void* stream) {
    LRKV_TRY(check_dims(dims));
    LRKV_TRY(check_cache(*dims, cache, true));
    LRKV_TRY(need_ptr(k_new, "k_new"));
    LRKV_TRY(need_ptr(v_new, "v_new"));
    if (dims->r > 0) {
        LRKV_TRY(need_ptr(zk_new, "zk_new"));
        LRKV_TRY(need_ptr(zv_new, "zv_new"));
    }
    hipError_t e = lrkv::launch_append(dims->batch, dims->H, dims->d_h, dims->r, dims->L_cap, dims->dtype,
                                       cache->k_shared, cache->v_shared, cache->z_k, cache->z_v, cache->seq_lens,
                                       k_new, v_new, zk_new, zv_new, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "append kernel launch");
    return ok();
}

lrkv_status lrkv_append_absorb(const lrkv_dims* dims, const lrkv_cache* cache, const void* k_new, const void* v_new,
                               const void* zk_new, const void* zv_new, const void* q, const void* B_k, float* p,
                               void* stream) {
    LRKV_TRY(check_dims(dims));
    if (dims->r == 0) return lrkv_cache_append(dims, cache, k_new, v_new, zk_new, zv_new, stream);
    LRKV_TRY(check_cache(*dims, cache, true));
    LRKV_TRY(need_ptr(k_new, "k_new"));
    LRKV_TRY(need_ptr(v_new, "v_new"));
    LRKV_TRY(need_ptr(zk_new, "zk_new"));
    LRKV_TRY(need_ptr(zv_new, "zv_new"));
    LRKV_TRY(need_ptr(q, "q"));
    LRKV_TRY(need_ptr(B_k, "B_k"));
    LRKV_TRY(need_ptr(p, "p"));
    if (!lrkv::append_absorb_supported(dims->H, dims->d_h, dims->r, dims->dtype)) {  // two launches
        LRKV_TRY(lrkv_cache_append(dims, cache, k_new, v_new, zk_new, zv_new, stream));
        return lrkv_absorb_query(dims, q, B_k, p, stream);
    }
    hipError_t e = lrkv::launch_append_absorb(dims->batch, dims->H, dims->d_h, dims->r, dims->L_cap, dims->dtype,
                                              cache->k_shared, cache->v_shared, cache->z_k, cache->z_v,
                                              cache->seq_lens, k_new, v_new, zk_new, zv_new, q, B_k, p,
                                              (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "append/absorb kernel launch");
    return ok();
}

lrkv_status lrkv_decode_partial(const lrkv_dims* dims, const lrkv_cache* cache, int32_t max_len, const void* q,
                                const float* p, void* workspace, size_t workspace_bytes_, void* stream) {
    lrkv::SplitPlan plan;
    LRKV_TRY(check_decode_common(dims, max_len, &plan));
    LRKV_TRY(check_cache(*dims, cache, true));
    LRKV_TRY(need_ptr(q, "q"));
    if (dims->r > 0) LRKV_TRY(need_ptr(p, "p"));
    LRKV_TRY(check_workspace(*dims, plan, workspace, workspace_bytes_));
    LRKV_TRY(run_partial(*dims, *cache, max_len, q, p, workspace, plan, (hipStream_t)stream));
    return ok();
}

lrkv_status lrkv_decode_merge(const lrkv_dims* dims, const int32_t* seq_lens, int32_t max_len, const void* B_v,
                              float* out, const void* workspace, size_t workspace_bytes_, void* stream) {
    lrkv::SplitPlan plan;
    LRKV_TRY(check_decode_common(dims, max_len, &plan));
    LRKV_TRY(need_ptr(seq_lens, "seq_lens"));
    LRKV_TRY(need_ptr(out, "out"));
    if (dims->r > 0) LRKV_TRY(need_ptr(B_v, "B_v"));
    LRKV_TRY(check_workspace(*dims, plan, workspace, workspace_bytes_));
    hipError_t e = lrkv::launch_merge(dims->batch, 1, 1, dims->H, dims->d_h, dims->r, dims->dtype, max_len, plan.chunk,
                                      plan.num_splits, seq_lens, B_v, out, (const float*)workspace,
                                      (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "merge kernel launch");
    return ok();
}

lrkv_status lrkv_decode(const lrkv_dims* dims, const lrkv_cache* cache, int32_t max_len, const void* q,
                        const float* p, const void* B_v, float* out, void* workspace, size_t workspace_bytes_,
                        void* stream) {
    lrkv::SplitPlan plan;
    LRKV_TRY(check_decode_common(dims, max_len, &plan));
    LRKV_TRY(check_cache(*dims, cache, true));
    LRKV_TRY(need_ptr(q, "q"));
    LRKV_TRY(need_ptr(out, "out"));
    if (dims->r > 0) {
        LRKV_TRY(need_ptr(p, "p"));
        LRKV_TRY(need_ptr(B_v, "B_v"));
    }
    LRKV_TRY(check_workspace(*dims, plan, workspace, workspace_bytes_));
    LRKV_TRY(run_partial(*dims, *cache, max_len, q, p, workspace, plan, (hipStream_t)stream));
    hipError_t e = lrkv::launch_merge(dims->batch, 1, 1, dims->H, dims->d_h, dims->r, dims->dtype, max_len, plan.chunk,
                                      plan.num_splits, cache->seq_lens, B_v, out, (const float*)workspace,
                                      (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "merge kernel launch");
    return ok();
}

lrkv_status lrkv_latents_to_token_major(const lrkv_dims* dims, const void* src, void* dst, void* stream) {
    LRKV_TRY(check_dims(dims));
    if (dims->r == 0) return ok();
    LRKV_TRY(need_ptr(src, "src"));
    LRKV_TRY(need_ptr(dst, "dst"));
    const size_t bytes = (size_t)dims->batch * dims->H * dims->L_cap * dims->r * (dims->dtype == LRKV_F32 ? 4 : 2);
    const uintptr_t s0 = reinterpret_cast<uintptr_t>(src), d0 = reinterpret_cast<uintptr_t>(dst);
    if (s0 < d0 + bytes && d0 < s0 + bytes) return fail(LRKV_ERR_INVALID_ARG, "src and dst overlap");
    hipError_t e = lrkv::launch_latents_token_major(dims->batch, dims->H, dims->L_cap, dims->r, dims->dtype, src, dst,
                                                    (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "latent layout kernel launch");
    return ok();
}

namespace {
// The fused step runs where the plain plan takes the bf16 matrix-core kernel, the absorb has its one-wave
// vector path (r == 0: no absorb) and the merge workgroups (one per (sequence, head), with the split kernel's
// registers) fit in one resident round: the 64-sequence ragged batch (2048 of them, four rounds at two per CU)
// ran 3% slower fused than as three launches.  On the fp32 rank-0 kernel (no absorb) the split pass appends the
// token and grows the lengths, and the merge kernel follows: two launches instead of three.
bool step_fused(const lrkv_dims& d, const lrkv::SplitPlan& plan) {
    if (plan.num_splits <= 0) return false;
    if (plan.path == lrkv::SplitPath::kMfmaF32) return true;
    return plan.path == lrkv::SplitPath::kMfmaBf16 &&
           (d.r == 0 || lrkv::absorb_wave_ok(d.d_h, d.r, 2)) && (long)d.batch * d.H <= 256L * plan.occupancy;
}
size_t round256(size_t x) { return (x + 255) & ~size_t(255); }
}  // namespace

size_t lrkv_decode_step_sync_offset(const lrkv_dims* dims, int32_t max_len) {
    if (!dims_valid(dims) || max_len < 0 || max_len > dims->L_cap) return 0;
    lrkv::SplitPlan p;
    if (!plan_split(*dims, max_len, &p)) return 0;
    return round256(workspace_bytes(*dims, p));
}

int32_t lrkv_decode_step_fused(const lrkv_dims* dims, int32_t max_len) {
    if (!dims_valid(dims) || max_len < 0 || max_len > dims->L_cap) return 0;
    lrkv::SplitPlan p;
    if (!plan_split(*dims, max_len, &p)) return 0;
    return step_fused(*dims, p) ? 1 : 0;
}

size_t lrkv_decode_step_workspace_bytes(const lrkv_dims* dims, int32_t max_len) {
    if (!dims_valid(dims) || max_len < 0 || max_len > dims->L_cap) return 0;
    lrkv::SplitPlan p;
    if (!plan_split(*dims, max_len, &p)) return 0;
    return round256(workspace_bytes(*dims, p)) + round256(sizeof(uint32_t) * lrkv::step_sync_words(dims->batch));
}

lrkv_status lrkv_decode_step(const lrkv_dims* dims, const lrkv_cache* cache, int32_t max_len, const void* k_new,
                             const void* v_new, const void* zk_new, const void* zv_new, const void* q,
                             const void* B_k, const void* B_v, float* p, float* out, void* workspace,
                             size_t workspace_bytes_, void* stream) {
    lrkv::SplitPlan plan;
    LRKV_TRY(check_decode_common(dims, max_len, &plan));
    LRKV_TRY(check_cache(*dims, cache, true));
    LRKV_TRY(need_ptr(k_new, "k_new"));
    LRKV_TRY(need_ptr(v_new, "v_new"));
    LRKV_TRY(need_ptr(q, "q"));
    LRKV_TRY(need_ptr(out, "out"));
    if (dims->r > 0) {
        LRKV_TRY(need_ptr(zk_new, "zk_new"));
        LRKV_TRY(need_ptr(zv_new, "zv_new"));
        LRKV_TRY(need_ptr(B_k, "B_k"));
        LRKV_TRY(need_ptr(B_v, "B_v"));
        LRKV_TRY(need_ptr(p, "p"));
    }
    const size_t need = lrkv_decode_step_workspace_bytes(dims, max_len);
    if (!workspace) return fail(LRKV_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", need);
    if (reinterpret_cast<uintptr_t>(workspace) & 255u) return fail(LRKV_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
    if (workspace_bytes_ < need) return fail(LRKV_ERR_WORKSPACE, "workspace has %zu bytes, need %zu", workspace_bytes_, need);
    if (!step_fused(*dims, plan)) {  // the two calls
        LRKV_TRY(lrkv_append_absorb(dims, cache, k_new, v_new, zk_new, zv_new, q, B_k, p, stream));
        return lrkv_decode(dims, cache, max_len, q, p, B_v, out, workspace, workspace_bytes_, stream);
    }
    using namespace lrkv;
    DecodeArgs a{};
    a.batch = dims->batch;
    a.H = dims->H;
    a.d_h = dims->d_h;
    a.r = dims->r;
    a.L_cap = dims->L_cap;
    a.dtype = dims->dtype;
    a.max_len = max_len;
    a.chunk = plan.chunk;
    a.num_splits = plan.num_splits;
    a.qgroup = 1;
    a.n_queries = 1;
    a.qw = 1;
    a.k_shared = cache->k_shared;
    a.v_shared = cache->v_shared;
    a.z_k = cache->z_k;
    a.z_v = cache->z_v;
    a.seq_lens = cache->seq_lens;
    a.seq_lens_rw = cache->seq_lens;
    a.q = q;
    a.p = p;
    a.p_out = p;
    a.ws = (float*)workspace;
    a.append_cap = dims->L_cap;
    a.n_absorb = dims->r > 0 ? (dims->batch * dims->H + 3) / 4 : 0;
    a.n_merge = dims->batch * dims->H;
    a.merge_wide = merge_wide(plan.num_splits, dims->batch) ? 1 : 0;
    a.k_new = k_new;
    a.v_new = v_new;
    a.zk_new = zk_new;
    a.zv_new = zv_new;
    a.B_k = B_k;
    a.B_v = B_v;
    a.out = out;
    a.sync = (uint32_t*)((char*)workspace + lrkv_decode_step_sync_offset(dims, max_len));
    if (plan.path == SplitPath::kMfmaF32) {
        // the split pass appends and grows the lengths; the merge reads the grown lengths (the pass's plan)
        hipError_t e = launch_step_mfma_f32(a, plan.occupancy, (hipStream_t)stream);
        if (e != hipSuccess) return hip_fail(e, "decode step split kernel launch");
        e = launch_merge(dims->batch, 1, 1, dims->H, dims->d_h, dims->r, dims->dtype, max_len, plan.chunk,
                         plan.num_splits, cache->seq_lens, B_v, out, (const float*)workspace, (hipStream_t)stream);
        if (e != hipSuccess) return hip_fail(e, "merge kernel launch");
        return ok();
    }
    const hipError_t e = launch_step_mfma(a, plan.occupancy, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "decode step kernel launch");
    return ok();
}

size_t lrkv_decode_noalloc_max_bytes(void) { return kScratchBytes; }

lrkv_status lrkv_decode_noalloc(const lrkv_dims* dims, const lrkv_cache* cache, int32_t max_len, const void* q,
                                const float* p, const void* B_v, float* out, void* stream) {
    lrkv::SplitPlan plan;
    LRKV_TRY(check_decode_common(dims, max_len, &plan));
    LRKV_TRY(check_cache(*dims, cache, true));
    LRKV_TRY(need_ptr(q, "q"));
    LRKV_TRY(need_ptr(out, "out"));
    if (dims->r > 0) {
        LRKV_TRY(need_ptr(p, "p"));
        LRKV_TRY(need_ptr(B_v, "B_v"));
    }
    const size_t need = workspace_bytes(*dims, plan);
    if (need > kScratchBytes)
        return fail(LRKV_ERR_WORKSPACE,
                    "lrkv_decode_noalloc: the split records need %zu bytes, more than its %zu-byte device scratch; "
                    "use lrkv_decode with a workspace",
                    need, kScratchBytes);
    void* ws = nullptr;  // no live rows anywhere (need == 0): the merge alone writes zeros, as in lrkv_decode
    hipError_t e = hipSuccess;
    if (need > 0) {
        // the device the stream belongs to (the current device for the null stream)
        int dev = -1;
        e = stream ? hipStreamGetDevice((hipStream_t)stream, &dev) : hipGetDevice(&dev);
        if (e != hipSuccess) return hip_fail(e, "lrkv_decode_noalloc: device of the stream");
        ws = scratch_on(dev, &e);
        if (!ws) return hip_fail(e, "lrkv_decode_noalloc: address of the device scratch");
    }
    LRKV_TRY(run_partial(*dims, *cache, max_len, q, p, ws, plan, (hipStream_t)stream));
    e = lrkv::launch_merge(dims->batch, 1, 1, dims->H, dims->d_h, dims->r, dims->dtype, max_len, plan.chunk,
                           plan.num_splits, cache->seq_lens, B_v, out, (const float*)ws, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "merge kernel launch");
    return ok();
}

}  // extern "C"

namespace {

// Multi-token decode runs as single-token decode of virtual sequences, each a set of qw consecutive query
// tokens of one cached sequence: set c of sequence b is virtual sequence b * nc + c (nc = ceil(Q / qw)) and
// reads sequence b's cache up to the causal length of its last token (token i sees seq_lens[b] - Q + 1 + i
// rows).  Shapes of the bf16 matrix-core kernel take qw = 2 (Q = 2) or 4 (Q >= 3): one workgroup serves the
// whole set from one read of the rows (qw = 2 at most for d_h = 128, r = 64, where four queries' state does
// not fit the registers).  Other shapes take qw = 1, one virtual sequence per token.  Tuning
// override (read at every call, so it must not change between a workspace query and the decode that uses it):
// LRKV_MULTI_QW (1, 2 or 4).  The workspace holds the plan's partial records ([G][qw][H][record]), then the
// virtual lengths (256-byte aligned parts).
struct MultiPlan {
    lrkv_dims dq;         // dims of the virtual batch
    lrkv::SplitPlan plan;
    int qw;               // query tokens per virtual sequence
    size_t records_bytes, total_bytes;
};

bool plan_multi(const lrkv_dims& d, int Q, int max_len, MultiPlan* mp) {
    if (Q < 1 || Q > 64 || (long long)d.batch * Q > 65535) return false;
    int qw = 1;
    if (Q > 1 && lrkv::mfma_path_supports(d.H, d.d_h, d.r, d.dtype, d.L_cap) &&
        lrkv::mfma_all_variants(d.H, d.d_h, d.r)) {
        const int qmax = lrkv::mfma_max_query_width(d.H, d.d_h, d.r);
        qw = env_int("LRKV_MULTI_QW", Q == 2 ? 2 : qmax);
        if (qw != 1 && qw != 2 && qw != 4) qw = qmax;
        qw = std::min(qw, qmax);
    }
    mp->qw = qw;
    mp->dq = d;
    mp->dq.batch = d.batch * ((Q + qw - 1) / qw);
    if (!plan_split(mp->dq, max_len, &mp->plan, qw > 1 ? PlanVariant::kQuerySets : PlanVariant::kPlain)) return false;
    if ((long long)mp->plan.num_splits * qw * d.H * lrkv::partial_record_floats(d.d_h, d.r) >= (1LL << 31))
        return false;  // the merge kernel addresses the records with 32-bit offsets
    mp->records_bytes = (qw * workspace_bytes(mp->dq, mp->plan) + 255) & ~(size_t)255;
    mp->total_bytes = mp->records_bytes + (((size_t)mp->dq.batch * sizeof(int32_t) + 255) & ~(size_t)255);
    return true;
}

}  // namespace

extern "C" {

size_t lrkv_decode_multi_workspace_bytes(const lrkv_dims* dims, int32_t n_queries, int32_t max_len) {
    if (!dims_valid(dims) || max_len < 0 || max_len > dims->L_cap) return 0;
    MultiPlan mp;
    if (!plan_multi(*dims, n_queries, max_len, &mp)) return 0;
    return mp.total_bytes;
}

lrkv_status lrkv_decode_multi(const lrkv_dims* dims, int32_t n_queries, const lrkv_cache* cache, int32_t max_len,
                              const void* q, const float* p, const void* B_v, float* out, void* workspace,
                              size_t workspace_bytes_, void* stream) {
    LRKV_TRY(check_dims(dims));
    if (max_len < 0 || max_len > dims->L_cap)
        return fail(LRKV_ERR_INVALID_ARG, "max_len=%d outside [0, L_cap=%d]", max_len, dims->L_cap);
    if (n_queries < 1 || n_queries > 64) return fail(LRKV_ERR_INVALID_ARG, "n_queries=%d outside [1, 64]", n_queries);
    MultiPlan mp;
    if (!plan_multi(*dims, n_queries, max_len, &mp))
        return fail(LRKV_ERR_UNSUPPORTED, "no kernel for batch*Q=%lld H=%d d_h=%d r=%d dtype=%d",
                    (long long)dims->batch * n_queries, dims->H, dims->d_h, dims->r, dims->dtype);
    LRKV_TRY(check_cache(*dims, cache, true));
    LRKV_TRY(need_ptr(q, "q"));
    LRKV_TRY(need_ptr(out, "out"));
    if (dims->r > 0) {
        LRKV_TRY(need_ptr(p, "p"));
        LRKV_TRY(need_ptr(B_v, "B_v"));
    }
    if (!workspace) return fail(LRKV_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", mp.total_bytes);
    if (reinterpret_cast<uintptr_t>(workspace) & 255u) return fail(LRKV_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
    if (workspace_bytes_ < mp.total_bytes)
        return fail(LRKV_ERR_WORKSPACE, "workspace has %zu bytes, need %zu", workspace_bytes_, mp.total_bytes);
    int32_t* vlens = (int32_t*)((char*)workspace + mp.records_bytes);
    hipError_t e =
        lrkv::launch_multi_lengths(dims->batch, n_queries, mp.qw, cache->seq_lens, vlens, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "length kernel launch");
    const lrkv_cache vc{cache->k_shared, cache->v_shared, cache->z_k, cache->z_v, vlens};
    QuerySets qs;
    qs.qgroup = (n_queries + mp.qw - 1) / mp.qw;
    qs.n_queries = n_queries;
    qs.qw = mp.qw;
    LRKV_TRY(run_partial(mp.dq, vc, max_len, q, p, workspace, mp.plan, (hipStream_t)stream, nullptr, PagedView(), qs));
    e = lrkv::launch_merge(dims->batch, n_queries, mp.qw, dims->H, dims->d_h, dims->r, dims->dtype, max_len,
                           mp.plan.chunk,
                           mp.plan.num_splits, vlens, B_v, out, (const float*)workspace, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "merge kernel launch");
    return ok();
}

lrkv_status lrkv_key_scales(const lrkv_dims* dims, const lrkv_cache* cache, int32_t max_len, int32_t n_last,
                            const void* B_k, float eps, void* rho, void* stream) {
    LRKV_TRY(check_dims(dims));
    if (max_len < 0 || max_len > dims->L_cap)
        return fail(LRKV_ERR_INVALID_ARG, "max_len=%d outside [0, L_cap=%d]", max_len, dims->L_cap);
    if (n_last < 0) return fail(LRKV_ERR_INVALID_ARG, "n_last=%d is negative", n_last);
    if (!(eps >= 0.f) || eps > 3.0e38f) return fail(LRKV_ERR_INVALID_ARG, "eps must be finite and >= 0");
    if (!cache) return fail(LRKV_ERR_INVALID_ARG, "cache is NULL");
    LRKV_TRY(need_ptr(cache->k_shared, "cache.k_shared"));
    LRKV_TRY(need_ptr(cache->seq_lens, "cache.seq_lens"));
    if (dims->r > 0) {
        LRKV_TRY(need_ptr(cache->z_k, "cache.z_k"));
        LRKV_TRY(need_ptr(B_k, "B_k"));
    }
    LRKV_TRY(need_ptr(rho, "rho"));
    hipError_t e = lrkv::launch_key_scales(dims->batch, dims->H, dims->d_h, dims->r, dims->L_cap, dims->dtype, max_len,
                                           n_last, eps, cache->seq_lens, cache->k_shared, cache->z_k, B_k, rho,
                                           (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "key scale kernel launch");
    return ok();
}

lrkv_status lrkv_norm_query(const lrkv_dims* dims, const void* q, const void* g_q, const void* g_k, float eps,
                            void* q_eff, void* stream) {
    LRKV_TRY(check_dims(dims));
    if (!(eps >= 0.f) || eps > 3.0e38f) return fail(LRKV_ERR_INVALID_ARG, "eps must be finite and >= 0");
    LRKV_TRY(need_ptr(q, "q"));
    LRKV_TRY(need_ptr(g_q, "g_q"));
    LRKV_TRY(need_ptr(g_k, "g_k"));
    LRKV_TRY(need_ptr(q_eff, "q_eff"));
    hipError_t e = lrkv::launch_norm_query(dims->batch, dims->H, dims->d_h, dims->dtype, eps, q, g_q, g_k, q_eff,
                                           (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "query normalisation kernel launch");
    return ok();
}

lrkv_status lrkv_decode_normed(const lrkv_dims* dims, const lrkv_cache* cache, const void* rho, int32_t max_len,
                               const void* q_eff, const float* p, const void* B_v, float* out, void* workspace,
                               size_t workspace_bytes_, void* stream) {
    lrkv::SplitPlan plan;
    LRKV_TRY(check_decode_common(dims, max_len, &plan, PlanVariant::kNormed));
    LRKV_TRY(check_cache(*dims, cache, true));
    LRKV_TRY(need_ptr(rho, "rho"));
    LRKV_TRY(need_ptr(q_eff, "q_eff"));
    LRKV_TRY(need_ptr(out, "out"));
    if (dims->r > 0) {
        LRKV_TRY(need_ptr(p, "p"));
        LRKV_TRY(need_ptr(B_v, "B_v"));
    }
    LRKV_TRY(check_workspace(*dims, plan, workspace, workspace_bytes_));
    LRKV_TRY(run_partial(*dims, *cache, max_len, q_eff, p, workspace, plan, (hipStream_t)stream, rho));
    hipError_t e = lrkv::launch_merge(dims->batch, 1, 1, dims->H, dims->d_h, dims->r, dims->dtype, max_len, plan.chunk,
                                      plan.num_splits, cache->seq_lens, B_v, out, (const float*)workspace,
                                      (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "merge kernel launch");
    return ok();
}

}  // extern "C"

namespace {

int log2_exact(int x) {  // log2 of a power of two, -1 otherwise
    if (x <= 0 || (x & (x - 1)) != 0) return -1;
    int k = 0;
    while ((1 << k) < x) ++k;
    return k;
}

lrkv_status check_paged(const lrkv_dims& d, const lrkv_paged_cache* c, PagedView* pv) {
    if (!c) return fail(LRKV_ERR_INVALID_ARG, "cache is NULL");
    LRKV_TRY(need_ptr(c->k_pages, "cache.k_pages"));
    LRKV_TRY(need_ptr(c->v_pages, "cache.v_pages"));
    LRKV_TRY(need_ptr(c->block_table, "cache.block_table"));
    LRKV_TRY(need_ptr(c->seq_lens, "cache.seq_lens"));
    if (d.r > 0) {
        LRKV_TRY(need_ptr(c->zk_pages, "cache.zk_pages"));
        LRKV_TRY(need_ptr(c->zv_pages, "cache.zv_pages"));
    }
    const int shift = log2_exact(c->page_rows);
    if (shift < 5) return fail(LRKV_ERR_INVALID_ARG, "page_rows=%d is not a power of two >= 32", c->page_rows);
    if (c->max_pages < 1 || c->n_pages < 1)
        return fail(LRKV_ERR_INVALID_ARG, "max_pages=%d and n_pages=%d must be >= 1", c->max_pages, c->n_pages);
    if ((long long)c->max_pages * c->page_rows != d.L_cap)
        return fail(LRKV_ERR_INVALID_ARG, "L_cap=%d differs from max_pages * page_rows = %lld", d.L_cap,
                    (long long)c->max_pages * c->page_rows);
    const long long s = d.dtype == LRKV_F32 ? 4 : 2;
    const long long pool_rows = (long long)c->n_pages * c->page_rows;
    if (pool_rows * d.d_h * s >= (1LL << 31) || pool_rows * d.H * d.r * s >= (1LL << 31))
        return fail(LRKV_ERR_UNSUPPORTED, "a page pool of %lld rows reaches 2^31 bytes", pool_rows);
    pv->block_table = c->block_table;
    pv->page_shift = shift;
    pv->max_pages = c->max_pages;
    pv->n_pages = c->n_pages;
    return LRKV_OK;
}

}  // namespace

extern "C" {

lrkv_status lrkv_paged_append(const lrkv_dims* dims, const lrkv_paged_cache* cache, const void* k_new,
                              const void* v_new, const void* zk_new, const void* zv_new, void* stream) {
    LRKV_TRY(check_dims(dims));
    PagedView pv;
    LRKV_TRY(check_paged(*dims, cache, &pv));
    LRKV_TRY(need_ptr(k_new, "k_new"));
    LRKV_TRY(need_ptr(v_new, "v_new"));
    if (dims->r > 0) {
        LRKV_TRY(need_ptr(zk_new, "zk_new"));
        LRKV_TRY(need_ptr(zv_new, "zv_new"));
    }
    hipError_t e = lrkv::launch_paged_append(dims->batch, dims->H, dims->d_h, dims->r, dims->dtype, pv.page_shift,
                                             pv.max_pages, cache->k_pages, cache->v_pages, cache->zk_pages,
                                             cache->zv_pages, cache->block_table, cache->seq_lens, k_new, v_new,
                                             zk_new, zv_new, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "paged append kernel launch");
    return ok();
}

lrkv_status lrkv_decode_paged(const lrkv_dims* dims, const lrkv_paged_cache* cache, int32_t max_len, const void* q,
                              const float* p, const void* B_v, float* out, void* workspace, size_t workspace_bytes_,
                              void* stream) {
    lrkv::SplitPlan plan;
    LRKV_TRY(check_decode_common(dims, max_len, &plan, PlanVariant::kPaged));
    PagedView pv;
    LRKV_TRY(check_paged(*dims, cache, &pv));
    LRKV_TRY(need_ptr(q, "q"));
    LRKV_TRY(need_ptr(out, "out"));
    if (dims->r > 0) {
        LRKV_TRY(need_ptr(p, "p"));
        LRKV_TRY(need_ptr(B_v, "B_v"));
    }
    LRKV_TRY(check_workspace(*dims, plan, workspace, workspace_bytes_));
    const lrkv_cache pools{cache->k_pages, cache->v_pages, cache->zk_pages, cache->zv_pages, cache->seq_lens};
    LRKV_TRY(run_partial(*dims, pools, max_len, q, p, workspace, plan, (hipStream_t)stream, nullptr, pv));
    hipError_t e = lrkv::launch_merge(dims->batch, 1, 1, dims->H, dims->d_h, dims->r, dims->dtype, max_len, plan.chunk,
                                      plan.num_splits, cache->seq_lens, B_v, out, (const float*)workspace,
                                      (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "merge kernel launch");
    return ok();
}

lrkv_status lrkv_read_probe(const void* src, size_t bytes, uint32_t* sink, void* stream) {
    LRKV_TRY(need_ptr(src, "src"));
    LRKV_TRY(need_ptr(sink, "sink"));
    if (bytes == 0 || bytes % 16 != 0) return fail(LRKV_ERR_INVALID_ARG, "bytes=%zu must be a positive multiple of 16", bytes);
    hipError_t e = lrkv::launch_read_probe(src, bytes, sink, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "read probe launch");
    return ok();
}

lrkv_status lrkv_rope_table(int32_t d_h, int32_t n_pos, float base, float* table, void* stream) {
    if (d_h < 2 || d_h > 4096 || (d_h & 1)) return fail(LRKV_ERR_INVALID_ARG, "d_h=%d must be even, 2..4096", d_h);
    if (n_pos < 0 || n_pos > (1 << 28)) return fail(LRKV_ERR_INVALID_ARG, "n_pos=%d outside [0, 2^28]", n_pos);
    if (!(base > 1.f) || base > 3.0e38f) return fail(LRKV_ERR_INVALID_ARG, "base must be finite and > 1");
    LRKV_TRY(need_ptr(table, "table"));
    hipError_t e = lrkv::launch_rope_table(d_h, n_pos, base, table, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "rotary table kernel launch");
    return ok();
}

size_t lrkv_decode_rope_workspace_bytes(const lrkv_dims* dims, int32_t max_len) {
    if (!dims_valid(dims) || max_len < 0 || max_len > dims->L_cap || dims->d_h % 4 != 0) return 0;
    lrkv::SplitPlan p;
    if (!plan_split(*dims, max_len, &p, PlanVariant::kRope)) return 0;
    return workspace_bytes(*dims, p);
}

lrkv_status lrkv_decode_rope(const lrkv_dims* dims, const lrkv_cache* cache, int32_t max_len, const void* q,
                             const void* B_k, const float* table, const void* B_v, float* out, void* workspace,
                             size_t workspace_bytes_, void* stream) {
    LRKV_TRY(check_dims(dims));
    if (dims->d_h % 4 != 0) return fail(LRKV_ERR_UNSUPPORTED, "rotary decode needs d_h a multiple of 4 (d_h=%d)", dims->d_h);
    lrkv::SplitPlan plan;
    LRKV_TRY(check_decode_common(dims, max_len, &plan, PlanVariant::kRope));
    LRKV_TRY(check_cache(*dims, cache, true));
    LRKV_TRY(need_ptr(q, "q"));
    LRKV_TRY(need_ptr(table, "table"));
    LRKV_TRY(need_ptr(out, "out"));
    if (dims->r > 0) {
        LRKV_TRY(need_ptr(B_k, "B_k"));
        LRKV_TRY(need_ptr(B_v, "B_v"));
    }
    LRKV_TRY(check_workspace(*dims, plan, workspace, workspace_bytes_));
    LRKV_TRY(run_partial(*dims, *cache, max_len, q, nullptr, workspace, plan, (hipStream_t)stream, nullptr,
                         PagedView(), QuerySets(), table, B_k));
    hipError_t e = lrkv::launch_merge(dims->batch, 1, 1, dims->H, dims->d_h, dims->r, dims->dtype, max_len, plan.chunk,
                                      plan.num_splits, cache->seq_lens, B_v, out, (const float*)workspace,
                                      (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "merge kernel launch");
    return ok();
}

lrkv_status lrkv_materialize(const lrkv_dims* dims, const lrkv_cache* cache, int32_t max_len, const void* B_k,
                             const void* B_v, void* K_out, void* V_out, void* stream) {
    LRKV_TRY(check_dims(dims));
    if (max_len < 0 || max_len > dims->L_cap)
        return fail(LRKV_ERR_INVALID_ARG, "max_len=%d outside [0, L_cap=%d]", max_len, dims->L_cap);
    LRKV_TRY(check_cache(*dims, cache, true));
    LRKV_TRY(need_ptr(K_out, "K_out"));
    LRKV_TRY(need_ptr(V_out, "V_out"));
    if (dims->r > 0) {
        LRKV_TRY(need_ptr(B_k, "B_k"));
        LRKV_TRY(need_ptr(B_v, "B_v"));
    }
    hipError_t e = lrkv::launch_materialize(dims->batch, dims->H, dims->d_h, dims->r, dims->L_cap, dims->dtype, max_len,
                                            cache->seq_lens, cache->k_shared, cache->v_shared, cache->z_k, cache->z_v,
                                            B_k, B_v, K_out, V_out, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "materialize kernel launch");
    return ok();
}

lrkv_status lrkv_project_append(const lrkv_dims* dims, int32_t d_model, const lrkv_cache* cache, const void* x,
                                const void* W_in, void* q_out, void* stream) {
    LRKV_TRY(check_dims(dims));
    if (d_model < 1) return fail(LRKV_ERR_INVALID_ARG, "d_model=%d must be >= 1", d_model);
    LRKV_TRY(check_cache(*dims, cache, true));
    LRKV_TRY(need_ptr(x, "x"));
    LRKV_TRY(need_ptr(W_in, "W_in"));
    LRKV_TRY(need_ptr(q_out, "q_out"));
    const long long n_in = (long long)dims->H * dims->d_h + 2LL * dims->d_h + 2LL * dims->H * dims->r;
    if (n_in * d_model >= (1LL << 31) || (long long)dims->batch * n_in >= (1LL << 31))
        return fail(LRKV_ERR_UNSUPPORTED, "projection of %lld features from d_model=%d is too large", n_in, d_model);
    hipError_t e = lrkv::launch_project_append(dims->batch, dims->H, dims->d_h, dims->r, dims->L_cap, dims->dtype,
                                               d_model, cache->k_shared, cache->v_shared, cache->z_k, cache->z_v,
                                               cache->seq_lens, x, W_in, q_out, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "projection kernel launch");
    return ok();
}

lrkv_status lrkv_output_project(const lrkv_dims* dims, int32_t d_model, const float* o, const void* W_o, float* y,
                                void* stream) {
    LRKV_TRY(check_dims(dims));
    if (d_model < 1) return fail(LRKV_ERR_INVALID_ARG, "d_model=%d must be >= 1", d_model);
    LRKV_TRY(need_ptr(o, "o"));
    LRKV_TRY(need_ptr(W_o, "W_o"));
    LRKV_TRY(need_ptr(y, "y"));
    const long long k = (long long)dims->H * dims->d_h;
    if (k * d_model >= (1LL << 31) || (long long)dims->batch * d_model >= (1LL << 31))
        return fail(LRKV_ERR_UNSUPPORTED, "output projection %lld x %d is too large", k, d_model);
    hipError_t e = lrkv::launch_output_project(dims->batch, dims->H, dims->d_h, dims->dtype, d_model, o, W_o, y,
                                               (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "output projection kernel launch");
    return ok();
}

}  // extern "C"
