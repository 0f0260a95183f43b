// Host side of the C ABI declared in include/kvpaged.h: pool and lease bookkeeping, argument
// checks done before any launch, and dispatch to the gfx950 kernels.
#include "../../include/kvpaged.h"
#include "internal.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <deque>
#include <mutex>
#include <string>
#include <vector>

struct kv_pool {
    int32_t num_pages, page_size, num_kv_heads, head_dim, max_streams;
    uint16_t *k_pages;
    uint16_t *v_pages;
    mutable std::mutex mu;
    std::deque<int32_t> free_q;
    std::vector<char> is_free;       // is_free[id]: id is in free_q
    std::vector<int32_t> holders;    // streams whose lease list holds id (0 for a free page)
    int32_t policy = KV_LEASE_QUEUE;
    std::vector<std::vector<int32_t>> leased;
};

namespace kvp {
// kernels_mfma.hip: whether the MFMA kernel a call of this shape runs writes and reads the
// call's own new rows itself (the direct-to-LDS kernel)
bool mfma_fuses_rows(int D, int P, int chunk);
}  // namespace kvp

namespace {

thread_local std::string g_last_error;
thread_local hipEvent_t g_part_start = nullptr;
thread_local hipEvent_t g_part_stop = nullptr;

kv_status fail(kv_status st, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

kv_status ok() { return KV_OK; }

bool check_enabled() {
    const char *e = getenv("KVP_CHECK");
    return e && e[0] && e[0] != '0';
}

int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

// The kernels move rows of q, out and new K/V in 16-byte pieces.
bool aligned16(const void *p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }

kv_status check_layout(const kv_pool *pool, const kv_layout *lay, const char *who) {
    if (!pool) return fail(KV_E_ARG, "%s: pool is null", who);
    if (!lay) return fail(KV_E_ARG, "%s: layout is null", who);
    if (lay->num_streams < 1) return fail(KV_E_ARG, "%s: num_streams %d < 1", who, lay->num_streams);
    if (lay->rows < 1) return fail(KV_E_ARG, "%s: rows %d < 1", who, lay->rows);
    if (!lay->page_table || !lay->seq_len) return fail(KV_E_ARG, "%s: page_table or seq_len is null", who);
    if (lay->max_seq_len < lay->rows)
        return fail(KV_E_ARG, "%s: max_seq_len %d < rows %d", who, lay->max_seq_len, lay->rows);
    if (lay->max_seq_len > KV_MAX_SEQ_LEN)
        return fail(KV_E_ARG, "%s: max_seq_len %d > %d", who, lay->max_seq_len, KV_MAX_SEQ_LEN);
    if (lay->ring_pages < 0) return fail(KV_E_ARG, "%s: ring_pages %d < 0", who, lay->ring_pages);
    const int need = lay->ring_pages ? lay->ring_pages : ceil_div(lay->max_seq_len, pool->page_size);
    if (lay->table_stride < need)
        return fail(KV_E_ARG, "%s: table_stride %d < %d entries needed for max_seq_len %d", who,
                    lay->table_stride, need, lay->max_seq_len);
    if ((int64_t)lay->num_streams * lay->rows > (int64_t)INT32_MAX / 4)
        return fail(KV_E_ARG, "%s: too many rows", who);
    return ok();
}

// Optional host validation of the device lengths and tables (KVP_CHECK=1).
// ring_span: how many consecutive positions one call needs the ring to hold (rows for a row
// write, window + rows - 1 for attention); ignored for full layers.
kv_status deep_check(const kv_pool *pool, const kv_layout *lay, int64_t ring_span, hipStream_t st, const char *who) {
    if (!check_enabled()) return ok();
    const int S = lay->num_streams;
    std::vector<int32_t> L(S), tab((size_t)S * lay->table_stride);
    if (hipMemcpyAsync(L.data(), lay->seq_len, sizeof(int32_t) * S, hipMemcpyDeviceToHost, st) != hipSuccess ||
        hipMemcpyAsync(tab.data(), lay->page_table, sizeof(int32_t) * tab.size(), hipMemcpyDeviceToHost, st) != hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess)
        return fail(KV_E_DEVICE, "%s: KVP_CHECK copy failed", who);
    for (int s = 0; s < S; ++s) {
        // a length below the row count is allowed: the rows at negative positions are skipped
        // by the row write and see no key in attention
        if (L[s] < 0 || L[s] > lay->max_seq_len)
            return fail(KV_E_ARG, "%s: stream %d has seq_len %d outside [0, max_seq_len %d]", who, s, L[s],
                        lay->max_seq_len);
        int n;
        if (lay->ring_pages) {
            n = lay->ring_pages;
            const int64_t cap = (int64_t)lay->ring_pages * pool->page_size;
            if (ring_span > cap)
                return fail(KV_E_ARG, "%s: a ring of %lld positions cannot hold the %lld a call needs", who,
                            (long long)cap, (long long)ring_span);
        } else {
            n = ceil_div(L[s], pool->page_size);
        }
        for (int i = 0; i < n; ++i) {
            const int32_t pg = tab[(size_t)s * lay->table_stride + i];
            if (pg < 0 || pg >= pool->num_pages)
                return fail(KV_E_ARG, "%s: stream %d table entry %d = %d outside [0, %d)", who, s, i, pg,
                            pool->num_pages);
        }
    }
    return ok();
}

struct Plan {
    int D, G, Hkv, Hq, S, R;
    kvp::CallPlan cp;
};

kv_status make_plan(const kv_pool *pool, const kv_layout *lay, const kv_attn_args *a, Plan *p, const char *who) {
    kv_status st = check_layout(pool, lay, who);
    if (st != KV_OK) return st;
    if (!a) return fail(KV_E_ARG, "%s: args is null", who);
    if (a->num_q_heads < 1 || a->num_q_heads % pool->num_kv_heads != 0)
        return fail(KV_E_ARG, "%s: num_q_heads %d is not a positive multiple of num_kv_heads %d", who,
                    a->num_q_heads, pool->num_kv_heads);
    if (a->window < 0 || a->window > KV_MAX_SEQ_LEN)
        return fail(KV_E_ARG, "%s: window %d outside [0, %d]", who, a->window, KV_MAX_SEQ_LEN);
    if (!(a->scale >= 0.f) || std::isinf(a->scale)) return fail(KV_E_ARG, "%s: scale must be finite and >= 0", who);
    if (lay->ring_pages && a->window <= 0)
        return fail(KV_E_ARG, "%s: a ring layer needs a sliding window", who);
    if (lay->ring_pages && (int64_t)a->window + lay->rows - 1 > (int64_t)lay->ring_pages * pool->page_size)
        return fail(KV_E_ARG, "%s: ring of %d pages x %d cannot hold window %d plus %d rows", who, lay->ring_pages,
                    pool->page_size, a->window, lay->rows);
    p->D = pool->head_dim;
    p->Hkv = pool->num_kv_heads;
    p->Hq = a->num_q_heads;
    p->G = p->Hq / p->Hkv;
    p->S = lay->num_streams;
    p->R = lay->rows;
    if (!kvp::call_plan(p->D, p->G, p->R, p->S, p->Hkv, pool->page_size, lay->max_seq_len, a->window, &p->cp))
        return fail(KV_E_SHAPE, "%s: no %s kernel for head_dim %d, group %d, rows %d", who,
                    p->R * p->G >= 16 ? "MFMA" : "VALU", p->D, p->G, p->R);
    return ok();
}

kvp::RowsArgs rows_args(const kv_pool *pool, const kv_layout *lay, const void *k_new, const void *v_new) {
    kvp::RowsArgs ra;
    ra.k_pages = pool->k_pages;
    ra.v_pages = pool->v_pages;
    ra.k_new = static_cast<const uint16_t *>(k_new);
    ra.v_new = static_cast<const uint16_t *>(v_new);
    ra.table = lay->page_table;
    ra.seq_len = lay->seq_len;
    ra.num_pages = pool->num_pages;
    ra.P = pool->page_size;
    ra.Hkv = pool->num_kv_heads;
    ra.D = pool->head_dim;
    ra.S = lay->num_streams;
    ra.R = lay->rows;
    ra.stride = lay->table_stride;
    ra.ring_pages = lay->ring_pages;
    ra.max_len = lay->max_seq_len;
    return ra;
}

size_t workspace_bytes(const Plan &p) {
    return (size_t)p.S * p.R * p.Hq * p.cp.n_splits * (p.D + 2) * sizeof(float);
}

kv_status run_attention(const kv_pool *pool, const kv_layout *lay, const kv_attn_args *a, void *hip_stream,
                        const char *who, const uint32_t *tree = nullptr, const void *k_new = nullptr,
                        const void *v_new = nullptr) {
    Plan p;
    kv_status st = make_plan(pool, lay, a, &p, who);
    if (st != KV_OK) return st;
    if (!a->q || !a->out) return fail(KV_E_ARG, "%s: q or out is null", who);
    if (!aligned16(a->q) || !aligned16(a->out)) return fail(KV_E_ARG, "%s: q and out must be 16-byte aligned", who);
    if ((k_new && !aligned16(k_new)) || (v_new && !aligned16(v_new)))
        return fail(KV_E_ARG, "%s: k_new and v_new must be 16-byte aligned", who);
    const size_t need = workspace_bytes(p);
    if (!a->workspace || a->workspace_bytes < need)
        return fail(KV_E_WORKSPACE, "%s: workspace of %zu bytes, %zu needed", who, a->workspace_bytes, need);
    if (reinterpret_cast<uintptr_t>(a->workspace) % 256 != 0)
        return fail(KV_E_ARG, "%s: workspace is not 256-byte aligned", who);
    hipStream_t hs = reinterpret_cast<hipStream_t>(hip_stream);
    st = deep_check(pool, lay, (int64_t)a->window + p.R - 1, hs, who);
    if (st != KV_OK) return st;

    kvp::PartArgs pa;
    pa.k_pages = pool->k_pages;
    pa.v_pages = pool->v_pages;
    pa.table = lay->page_table;
    pa.seq_len = lay->seq_len;
    pa.q = static_cast<const uint16_t *>(a->q);
    pa.ws_acc = static_cast<float *>(a->workspace);
    pa.ws_ml = pa.ws_acc + (size_t)p.S * p.R * p.Hq * p.cp.n_splits * p.D;
    pa.num_pages = pool->num_pages;
    pa.P = pool->page_size;
    pa.Hkv = p.Hkv;
    pa.stride = lay->table_stride;
    pa.ring_pages = lay->ring_pages;
    pa.max_len = lay->max_seq_len;
    pa.R = p.R;
    pa.Hq = p.Hq;
    pa.window = a->window;
    pa.n_splits = p.cp.n_splits;
    pa.chunk = p.cp.chunk;
    pa.out = static_cast<uint16_t *>(a->out);
    pa.tree = tree;
    pa.k_new = static_cast<const uint16_t *>(k_new);
    pa.v_new = static_cast<const uint16_t *>(v_new);
    pa.direct = (p.cp.mfma && p.cp.mp.direct) ? 1 : 0;
    const float scale = a->scale > 0.f ? a->scale : 1.0f / std::sqrt((float)p.D);
    pa.scale_log2 = scale * 1.4426950408889634f;

    // The new rows go in with the attention where its kernel writes them itself: the VALU
    // kernel for one row per stream, the direct-to-LDS MFMA kernel for any rows.  Otherwise
    // they go in first with the row-write kernel, on the same stream, so that the attention
    // reads them as kv_rows_put leaves them.
    const bool fused = p.cp.mfma ? kvp::mfma_fuses_rows(p.D, pool->page_size, p.cp.mp.chunk) : p.R == 1;
    if (k_new && !fused) {
        pa.k_new = pa.v_new = nullptr;
        const hipError_t e = kvp::launch_rows_put(rows_args(pool, lay, k_new, v_new), hs);
        if (e != hipSuccess) return fail(KV_E_DEVICE, "%s: row-write launch failed: %s", who, hipGetErrorString(e));
    }
    if (g_part_start && hipEventRecord(g_part_start, hs) != hipSuccess)
        return fail(KV_E_DEVICE, "%s: recording the start event failed", who);
    hipError_t e = p.cp.mfma ? kvp::launch_part_mfma(p.D, p.G, p.cp.mp, pa, p.S, hs)
                          : kvp::launch_part_valu(p.D, p.G, p.R * p.G, pa, p.S, hs);
    if (e != hipSuccess) return fail(KV_E_DEVICE, "%s: part kernel launch failed: %s", who, hipGetErrorString(e));
    if (g_part_stop && hipEventRecord(g_part_stop, hs) != hipSuccess)
        return fail(KV_E_DEVICE, "%s: recording the stop event failed", who);

    if (pa.direct) return ok();    // the part kernel wrote the output

    kvp::MergeArgs ma;
    ma.ws_acc = pa.ws_acc;
    ma.ws_ml = pa.ws_ml;
    ma.seq_len = lay->seq_len;
    ma.out = static_cast<uint16_t *>(a->out);
    ma.S = p.S;
    ma.R = p.R;
    ma.Hq = p.Hq;
    ma.D = p.D;
    ma.window = a->window;
    ma.max_len = lay->max_seq_len;
    ma.n_splits = p.cp.n_splits;
    ma.chunk = p.cp.chunk;
    ma.even = p.cp.even ? 1 : 0;
    ma.align = p.cp.align;
    e = kvp::launch_merge(ma, hs);
    if (e != hipSuccess) return fail(KV_E_DEVICE, "%s: merge launch failed: %s", who, hipGetErrorString(e));
    return ok();
}

// The ids KV_LEASE_CONTIGUOUS hands out for a lease of n (1 <= n <= free count) to a stream
// holding `held`: its own run extended, else a place in the longest free run that fits, else
// the lowest free ids.
std::vector<int32_t> contiguous_pick(const kv_pool *pool, const std::vector<int32_t> &held, int32_t n) {
    const int32_t N = pool->num_pages;
    const auto &fr = pool->is_free;
    std::vector<int32_t> got;
    got.reserve(n);
    if (!held.empty()) {
        const int64_t t = held.back();
        bool room = t + n < N;
        for (int64_t i = t + 1; room && i <= t + n; ++i) room = fr[i] != 0;
        if (room) {
            for (int32_t i = 1; i <= n; ++i) got.push_back((int32_t)(t + i));
            return got;
        }
    }
    int32_t best_a = -1, best_len = 0;
    for (int32_t a = 0; a < N;) {
        if (!fr[a]) {
            ++a;
            continue;
        }
        int32_t b = a;
        while (b < N && fr[b]) ++b;
        if (b - a >= n && b - a > best_len) {
            best_a = a;
            best_len = b - a;
        }
        a = b;
    }
    if (best_a >= 0) {
        const int32_t start = best_a == 0 ? 0 : best_a + (best_len - n) / 2;
        for (int32_t i = 0; i < n; ++i) got.push_back(start + i);
        return got;
    }
    for (int32_t id = 0; id < N && (int32_t)got.size() < n; ++id)
        if (fr[id]) got.push_back(id);
    return got;
}

}  // namespace

namespace kvp {

// Splits of an MFMA call that is not direct: the chunks from the first one any row of a stream
// sees to the stream's end (max_seq_len bounds the end; a window bounds the count).
static int splits_for(int max_seq_len, int rows, int window, int chunk) {
    int n = (int)(((int64_t)max_seq_len + chunk - 1) / chunk);
    if (window > 0) {
        const int span = (int)(((int64_t)window + rows - 1 + chunk - 1) / chunk) + 1;
        if (span < n) n = span;
    }
    return n < 1 ? 1 : n;
}

bool call_plan(int D, int G, int R, int S, int Hkv, int P, int max_seq_len, int window, CallPlan *p) {
    const int nq = R * G;
    p->mfma = nq >= 16;
    if (p->mfma) {
        if (!mfma_supported(D, G, R)) return false;
        p->mp = mfma_plan(D, G, R, S, Hkv, P, max_seq_len, window);
        p->chunk = p->mp.chunk;
        p->n_splits = p->mp.direct ? 1 : splits_for(max_seq_len, R, window, p->chunk);
        p->even = false;
        p->align = 1;
        return true;
    }
    if (!valu_supported(D, G, nq)) return false;
    // L - base is at most max_seq_len, or the window plus the rows plus the alignment
    int span = max_seq_len;
    const int align = valu_batch_keys(D);
    if (window > 0 && (int64_t)window + R - 1 + align - 1 < span) span = window + R - 1 + align - 1;
    const ValuPlan vp = valu_plan(D, nq, S, Hkv, span < 1 ? 1 : span);
    p->mp = MfmaPlan{};
    p->chunk = vp.max_piece;
    p->n_splits = vp.n_splits;
    p->even = true;
    p->align = vp.align;
    return true;
}

}  // namespace kvp

extern "C" {

kv_status kv_pool_create(const kv_pool_desc *d, kv_pool **out) {
    if (!d || !out) return fail(KV_E_ARG, "kv_pool_create: desc or out is null");
    if (d->num_pages < 1 || d->page_size < 1 || d->num_kv_heads < 1 || d->head_dim < 8 || d->max_streams < 1)
        return fail(KV_E_ARG, "kv_pool_create: sizes must be positive (num_pages %d, page_size %d, kv_heads %d, "
                    "head_dim %d, max_streams %d)", d->num_pages, d->page_size, d->num_kv_heads, d->head_dim,
                    d->max_streams);
    if (d->head_dim % 8 != 0) return fail(KV_E_ARG, "kv_pool_create: head_dim %d is not a multiple of 8", d->head_dim);
    if (!d->k_pages || !d->v_pages) return fail(KV_E_ARG, "kv_pool_create: k_pages or v_pages is null");
    if ((reinterpret_cast<uintptr_t>(d->k_pages) | reinterpret_cast<uintptr_t>(d->v_pages)) % 16 != 0)
        return fail(KV_E_ARG, "kv_pool_create: page arrays must be 16-byte aligned");
    std::vector<int32_t> order(d->num_pages);
    if (d->free_order) {
        std::vector<char> seen(d->num_pages, 0);
        for (int i = 0; i < d->num_pages; ++i) {
            const int32_t id = d->free_order[i];
            if (id < 0 || id >= d->num_pages || seen[id])
                return fail(KV_E_ARG, "kv_pool_create: free_order is not a permutation of [0, %d)", d->num_pages);
            seen[id] = 1;
            order[i] = id;
        }
    } else {
        for (int i = 0; i < d->num_pages; ++i) order[i] = i;
    }
    kv_pool *p = new (std::nothrow) kv_pool;
    if (!p) return fail(KV_E_ARG, "kv_pool_create: out of host memory");
    p->num_pages = d->num_pages;
    p->page_size = d->page_size;
    p->num_kv_heads = d->num_kv_heads;
    p->head_dim = d->head_dim;
    p->max_streams = d->max_streams;
    p->k_pages = static_cast<uint16_t *>(d->k_pages);
    p->v_pages = static_cast<uint16_t *>(d->v_pages);
    p->free_q.assign(order.begin(), order.end());
    p->is_free.assign(d->num_pages, 1);
    p->holders.assign(d->num_pages, 0);
    p->leased.assign(d->max_streams, {});
    *out = p;
    return ok();
}

kv_status kv_pool_destroy(kv_pool *pool) {
    delete pool;
    return ok();
}

kv_status kv_page_lease(kv_pool *pool, int32_t stream, int32_t n, int32_t *ids) {
    if (!pool) return fail(KV_E_ARG, "kv_page_lease: pool is null");
    std::lock_guard<std::mutex> lk(pool->mu);
    if (stream < 0 || stream >= pool->max_streams)
        return fail(KV_E_ARG, "kv_page_lease: stream %d outside [0, %d)", stream, pool->max_streams);
    if (n < 0) return fail(KV_E_ARG, "kv_page_lease: n %d < 0", n);
    if (n > 0 && !ids) return fail(KV_E_ARG, "kv_page_lease: page_ids_out is null");
    if ((size_t)n > pool->free_q.size())
        return fail(KV_E_NO_PAGES, "kv_page_lease: %d pages asked, %zu free", n, pool->free_q.size());
    auto &lst = pool->leased[stream];
    if (n == 0) return ok();
    if (pool->policy == KV_LEASE_QUEUE) {
        for (int i = 0; i < n; ++i) {
            ids[i] = pool->free_q.front();
            pool->free_q.pop_front();
            pool->is_free[ids[i]] = 0;
            pool->holders[ids[i]] = 1;
            lst.push_back(ids[i]);
        }
        return ok();
    }
    const std::vector<int32_t> got = contiguous_pick(pool, lst, n);
    for (int i = 0; i < n; ++i) {
        ids[i] = got[i];
        pool->is_free[got[i]] = 0;
        pool->holders[got[i]] = 1;
        lst.push_back(got[i]);
    }
    auto &q = pool->free_q;
    q.erase(std::remove_if(q.begin(), q.end(), [&](int32_t id) { return !pool->is_free[id]; }), q.end());
    return ok();
}

kv_status kv_pool_set_lease_policy(kv_pool *pool, int32_t policy) {
    if (!pool) return fail(KV_E_ARG, "kv_pool_set_lease_policy: pool is null");
    if (policy != KV_LEASE_QUEUE && policy != KV_LEASE_CONTIGUOUS)
        return fail(KV_E_ARG, "kv_pool_set_lease_policy: unknown policy %d", policy);
    std::lock_guard<std::mutex> lk(pool->mu);
    pool->policy = policy;
    return ok();
}

kv_status kv_page_release(kv_pool *pool, int32_t stream) {
    if (!pool) return fail(KV_E_ARG, "kv_page_release: pool is null");
    std::lock_guard<std::mutex> lk(pool->mu);
    if (stream < 0 || stream >= pool->max_streams)
        return fail(KV_E_ARG, "kv_page_release: stream %d outside [0, %d)", stream, pool->max_streams);
    auto &lst = pool->leased[stream];
    for (int32_t id : lst) {
        if (--pool->holders[id] > 0) continue;     // another stream still holds it
        pool->free_q.push_back(id);
        pool->is_free[id] = 1;
    }
    lst.clear();
    return ok();
}

kv_status kv_page_share(kv_pool *pool, int32_t src_stream, int32_t dst_stream, int32_t n) {
    if (!pool) return fail(KV_E_ARG, "kv_page_share: pool is null");
    std::lock_guard<std::mutex> lk(pool->mu);
    if (src_stream < 0 || src_stream >= pool->max_streams || dst_stream < 0 || dst_stream >= pool->max_streams)
        return fail(KV_E_ARG, "kv_page_share: stream %d or %d outside [0, %d)", src_stream, dst_stream,
                    pool->max_streams);
    if (src_stream == dst_stream) return fail(KV_E_ARG, "kv_page_share: a stream cannot share with itself");
    const auto &src = pool->leased[src_stream];
    auto &dst = pool->leased[dst_stream];
    if (n < 0 || (size_t)n > src.size())
        return fail(KV_E_ARG, "kv_page_share: n %d outside [0, %zu]", n, src.size());
    if (!dst.empty()) return fail(KV_E_ARG, "kv_page_share: stream %d already holds pages", dst_stream);
    for (int32_t i = 0; i < n; ++i) {
        dst.push_back(src[i]);
        ++pool->holders[src[i]];
    }
    return ok();
}

kv_status kv_pool_free_count(const kv_pool *pool, int32_t *out) {
    if (!pool || !out) return fail(KV_E_ARG, "kv_pool_free_count: null argument");
    std::lock_guard<std::mutex> lk(pool->mu);
    *out = (int32_t)pool->free_q.size();
    return ok();
}

kv_status kv_stream_pages(const kv_pool *pool, int32_t stream, int32_t *ids_out, int32_t cap, int32_t *n_out) {
    if (!pool || !n_out) return fail(KV_E_ARG, "kv_stream_pages: null argument");
    std::lock_guard<std::mutex> lk(pool->mu);
    if (stream < 0 || stream >= pool->max_streams)
        return fail(KV_E_ARG, "kv_stream_pages: stream %d outside [0, %d)", stream, pool->max_streams);
    if (cap < 0 || (cap > 0 && !ids_out)) return fail(KV_E_ARG, "kv_stream_pages: bad output buffer");
    const auto &lst = pool->leased[stream];
    const int n = (int)lst.size();
    for (int i = 0; i < n && i < cap; ++i) ids_out[i] = lst[i];
    *n_out = n;
    return ok();
}

kv_status kv_pages_copy(const kv_pool *pool, const int32_t *src_ids, const int32_t *dst_ids, int32_t n,
                        void *hip_stream) {
    if (!pool) return fail(KV_E_ARG, "kv_pages_copy: pool is null");
    if (n < 0) return fail(KV_E_ARG, "kv_pages_copy: n %d < 0", n);
    if (n == 0) return ok();
    if (!src_ids || !dst_ids) return fail(KV_E_ARG, "kv_pages_copy: src_ids or dst_ids is null");
    hipStream_t hs = reinterpret_cast<hipStream_t>(hip_stream);
    if (check_enabled()) {
        std::vector<int32_t> src(n), dst(n);
        if (hipMemcpyAsync(src.data(), src_ids, sizeof(int32_t) * n, hipMemcpyDeviceToHost, hs) != hipSuccess ||
            hipMemcpyAsync(dst.data(), dst_ids, sizeof(int32_t) * n, hipMemcpyDeviceToHost, hs) != hipSuccess ||
            hipStreamSynchronize(hs) != hipSuccess)
            return fail(KV_E_DEVICE, "kv_pages_copy: KVP_CHECK copy failed");
        std::vector<char> is_src(pool->num_pages, 0), is_dst(pool->num_pages, 0);
        for (int i = 0; i < n; ++i) {
            if (src[i] < 0 || src[i] >= pool->num_pages || dst[i] < 0 || dst[i] >= pool->num_pages)
                return fail(KV_E_ARG, "kv_pages_copy: pair %d (%d -> %d) outside [0, %d)", i, src[i], dst[i],
                            pool->num_pages);
            if (is_dst[dst[i]]) return fail(KV_E_ARG, "kv_pages_copy: page %d is a destination twice", dst[i]);
            is_src[src[i]] = 1;
            is_dst[dst[i]] = 1;
        }
        for (int i = 0; i < n; ++i)
            if (is_src[dst[i]]) return fail(KV_E_ARG, "kv_pages_copy: page %d is both a source and a destination", dst[i]);
    }
    kvp::CopyArgs ca;
    ca.k_pages = pool->k_pages;
    ca.v_pages = pool->v_pages;
    ca.src = src_ids;
    ca.dst = dst_ids;
    ca.n = n;
    ca.num_pages = pool->num_pages;
    ca.page_elems = (size_t)pool->num_kv_heads * pool->page_size * pool->head_dim;
    const hipError_t e = kvp::launch_pages_copy(ca, hs);
    if (e != hipSuccess) return fail(KV_E_DEVICE, "kv_pages_copy: launch failed: %s", hipGetErrorString(e));
    return ok();
}

kv_status kv_rows_put(const kv_pool *pool, const kv_layout *lay, const void *k_new, const void *v_new,
                      void *hip_stream) {
    kv_status st = check_layout(pool, lay, "kv_rows_put");
    if (st != KV_OK) return st;
    if (!k_new || !v_new) return fail(KV_E_ARG, "kv_rows_put: k_new or v_new is null");
    if (!aligned16(k_new) || !aligned16(v_new)) return fail(KV_E_ARG, "kv_rows_put: k_new and v_new must be 16-byte aligned");
    hipStream_t hs = reinterpret_cast<hipStream_t>(hip_stream);
    if (lay->ring_pages && (int64_t)lay->rows > (int64_t)lay->ring_pages * pool->page_size)
        return fail(KV_E_ARG, "kv_rows_put: %d rows overrun a ring of %d x %d positions", lay->rows,
                    lay->ring_pages, pool->page_size);
    st = deep_check(pool, lay, lay->rows, hs, "kv_rows_put");
    if (st != KV_OK) return st;
    const hipError_t e = kvp::launch_rows_put(rows_args(pool, lay, k_new, v_new), hs);
    if (e != hipSuccess) return fail(KV_E_DEVICE, "kv_rows_put: launch failed: %s", hipGetErrorString(e));
    return ok();
}

kv_status paged_attn_workspace_size(const kv_pool *pool, const kv_layout *lay, const kv_attn_args *a,
                                    size_t *bytes) {
    if (!bytes) return fail(KV_E_ARG, "paged_attn_workspace_size: bytes is null");
    Plan p;
    kv_status st = make_plan(pool, lay, a, &p, "paged_attn_workspace_size");
    if (st != KV_OK) return st;
    *bytes = workspace_bytes(p);
    return ok();
}

kv_status paged_attn_decode(const kv_pool *pool, const kv_layout *lay, const kv_attn_args *a, void *hip_stream) {
    if (lay && lay->rows != 1) return fail(KV_E_ARG, "paged_attn_decode: rows %d != 1", lay->rows);
    return run_attention(pool, lay, a, hip_stream, "paged_attn_decode");
}

kv_status paged_attn_decode_put(const kv_pool *pool, const kv_layout *lay, const kv_attn_args *a,
                                const void *k_new, const void *v_new, void *hip_stream) {
    if (lay && lay->rows != 1) return fail(KV_E_ARG, "paged_attn_decode_put: rows %d != 1", lay->rows);
    if (!k_new || !v_new) return fail(KV_E_ARG, "paged_attn_decode_put: k_new or v_new is null");
    return run_attention(pool, lay, a, hip_stream, "paged_attn_decode_put", nullptr, k_new, v_new);
}

kv_status paged_attn_decode_put_static(const kv_pool *pool, const kv_layout *lay, const kv_attn_args *a,
                                       const void *k_new, const void *v_new, void *hip_stream) {
    const char *who = "paged_attn_decode_put_static";
    if (lay && lay->rows != 1) return fail(KV_E_ARG, "%s: rows %d != 1", who, lay->rows);
    if (!k_new || !v_new) return fail(KV_E_ARG, "%s: k_new or v_new is null", who);
    Plan p;
    kv_status st = make_plan(pool, lay, a, &p, who);
    if (st != KV_OK) return st;
    const size_t need = workspace_bytes(p);
    if (need > (size_t)KV_STATIC_SCRATCH_BYTES)
        return fail(KV_E_WORKSPACE, "%s: the call needs %zu bytes of scratch, more than the %zu the library holds",
                    who, need, (size_t)KV_STATIC_SCRATCH_BYTES);
    void *ptr = nullptr;
    size_t have = 0;
    const hipError_t e = kvp::static_scratch(&ptr, &have);
    if (e != hipSuccess) return fail(KV_E_DEVICE, "%s: looking up the scratch array failed: %s", who, hipGetErrorString(e));
    kv_attn_args b = *a;
    b.workspace = ptr;
    b.workspace_bytes = have;
    return run_attention(pool, lay, &b, hip_stream, who, nullptr, k_new, v_new);
}

kv_status paged_attn_verify(const kv_pool *pool, const kv_layout *lay, const kv_attn_args *a, void *hip_stream) {
    if (lay && (lay->rows < 1 || lay->rows > 8))
        return fail(KV_E_ARG, "paged_attn_verify: rows %d outside 1..8", lay->rows);
    return run_attention(pool, lay, a, hip_stream, "paged_attn_verify");
}

kv_status paged_attn_verify_tree(const kv_pool *pool, const kv_layout *lay, const kv_attn_args *a,
                                 const uint32_t *tree_mask, void *hip_stream) {
    if (lay && (lay->rows < 1 || lay->rows > 8))
        return fail(KV_E_ARG, "paged_attn_verify_tree: rows %d outside 1..8", lay->rows);
    if (!tree_mask) return fail(KV_E_ARG, "paged_attn_verify_tree: tree_mask is null");
    return run_attention(pool, lay, a, hip_stream, "paged_attn_verify_tree", tree_mask);
}

kv_status paged_attn_prefill(const kv_pool *pool, const kv_layout *lay, const kv_attn_args *a, void *hip_stream) {
    if (lay && lay->rows < 1) return fail(KV_E_ARG, "paged_attn_prefill: rows %d < 1", lay->rows);
    return run_attention(pool, lay, a, hip_stream, "paged_attn_prefill");
}

kv_status paged_attn_prefill_put(const kv_pool *pool, const kv_layout *lay, const kv_attn_args *a,
                                 const void *k_new, const void *v_new, void *hip_stream) {
    if (lay && lay->rows < 1) return fail(KV_E_ARG, "paged_attn_prefill_put: rows %d < 1", lay->rows);
    if (!k_new || !v_new) return fail(KV_E_ARG, "paged_attn_prefill_put: k_new or v_new is null");
    return run_attention(pool, lay, a, hip_stream, "paged_attn_prefill_put", nullptr, k_new, v_new);
}

kv_status kv_set_part_events(void *start_event, void *stop_event) {
    if ((start_event == nullptr) != (stop_event == nullptr))
        return fail(KV_E_ARG, "kv_set_part_events: give both events or neither");
    g_part_start = static_cast<hipEvent_t>(start_event);
    g_part_stop = static_cast<hipEvent_t>(stop_event);
    return ok();
}

const char *kv_last_error(void) { return g_last_error.c_str(); }

int32_t kv_abi_version(void) { return KVPAGED_ABI_VERSION; }

}  // extern "C"
