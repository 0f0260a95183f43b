// Host check of the attention kernels' key ranges and page lookups, run without a GPU.
//
// For many call shapes (head dim, GQA group, rows, page size, max_seq_len, window, ring,
// table stride) and device lengths (edges, random values, and lengths above max_seq_len,
// which are caller errors), the checker takes the library's own launch plan (kvp::call_plan)
// and the functions the kernels themselves use for their key ranges, lookup modes and merge
// spans (internal.h), and walks every workgroup's load steps in the order the kernels issue
// them.  It checks that
//   * every page a load step reads is inside the pool and every row offset inside its page;
//   * every key a workgroup uses maps, through its cached or global table entries, to the
//     page the stream's table gives for that position (a cached index never falls outside the
//     cache for a key that is used);
//   * the pieces (VALU) or chunks (MFMA, per query tile) of a stream cover the keys its rows
//     see exactly once;
//   * the merge of each row combines only splits that were written and that hold all of the
//     row's keys;
//   * the fused decode row write finds the page of position L - 1;
//   * with a prompt chunk's row write fused into the MFMA kernel, every new row is written by
//     exactly one workgroup, into the page the table gives for its position, and no key a
//     workgroup reads from the pages shares its slot with a row the call writes;
//   * a device length above max_seq_len is read as max_seq_len.
// Streams at the longest length a call may describe (KV_MAX_SEQ_LEN) are checked for their
// ranges and merge spans only (no row walk): the checker is built with the signed-overflow
// check of UndefinedBehaviorSanitizer, so any 32-bit overflow in the shared range functions
// aborts it.
// `--plant merge` drops the last split of every merge span, `--plant cache` shrinks the
// checker's idea of the table cache by one entry and `--plant put` starts each tile's fused
// row write one row late: each must be reported.  `--plant overflow`
// feeds split_piece a length past the limit: the sanitizer must stop the run.
//
// Exit status 0 and a line "violations 0" when every check holds.
#include "../include/kvpaged.h"
#include "internal.h"

#include <algorithm>
#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <string>
#include <vector>

using namespace kvp;

namespace kvp {
// kernels_mfma.hip: whether a call of this shape runs the kernel that writes its own new rows
bool mfma_fuses_rows(int D, int P, int chunk);
}  // namespace kvp

namespace {

struct Shape {
    int D, G, R, S, Hkv, P, max_len, window, ring, extra_stride;
};

std::string plant;
bool walk_rows = true;      // false: ranges and merge spans only (streams too long to walk)
long long violations = 0, wg_checked = 0, rows_checked = 0, lengths_checked = 0;
long long fallbacks = 0;   // rows read through an absent entry (page 0), none of them used
long long outside = 0;     // lookups whose index falls outside the cache (the guard's case)

void report(const Shape &c, int L, const char *what, long long a, long long b) {
    ++violations;
    if (violations <= 20)
        std::printf("VIOLATION %s: D %d G %d R %d S %d P %d max %d W %d ring %d stride+%d L %d (%lld, %lld)\n", what,
                    c.D, c.G, c.R, c.S, c.P, c.max_len, c.window, c.ring, c.extra_stride, L, a, b);
}

// The stream's table: entries [0, stride), pages of a pool of num_pages (entries are only
// filled in when rows are walked).
struct Table {
    std::vector<int32_t> e;
    int num_pages;
    int stride;
};

Table make_table(int stride, uint32_t seed) {
    Table t;
    t.num_pages = 2 * stride + 5;
    t.stride = stride;
    if (!walk_rows) return t;
    t.e.resize(stride);
    for (int i = 0; i < stride; ++i) t.e[i] = (int32_t)((seed + 7919u * (uint32_t)i) % (uint32_t)t.num_pages);
    return t;
}

int cache_entries() { return plant == "cache" ? kTableCache - 1 : kTableCache; }

// The page the stream's table gives for position j (0 <= j < L <= max_len).
int true_page(const Shape &c, const Table &t, int j) {
    int idx = j / c.P;
    if (c.ring) idx %= c.ring;
    return t.e[idx];
}

// Entries a workgroup caches: logical pages idx0 + i (mod ring), -1 past the table or outside
// the pool.
std::vector<int> cached_entries(const Shape &c, const Table &t, bool whole, int idx0) {
    std::vector<int> v(kTableCache);
    const int stride = t.stride;
    for (int i = 0; i < kTableCache; ++i) {
        int idx = whole ? i : idx0 + i;
        if (!whole && c.ring) idx %= c.ring;
        const int pg = idx < stride ? t.e[idx] : -1;
        v[i] = (pg >= 0 && pg < t.num_pages) ? pg : -1;
    }
    return v;
}

// A page lookup as the kernels make it: the page read, and whether it came from an absent
// entry (an index outside the cache or the table, or an entry outside the pool: page 0).
struct Lookup {
    int pg;
    bool absent;
};

Lookup cached_page(const std::vector<int> &t, int i) {
    if ((unsigned)i >= (unsigned)cache_entries()) {
        ++outside;
        return {0, true};
    }
    if (t[i] < 0) return {0, true};
    return {t[i], false};
}

Lookup global_page(const Shape &c, const Table &t, int idx) {
    if (c.ring) idx %= c.ring;
    const int stride = t.stride;
    const int tp = t.e[std::min(idx, stride - 1)];
    if (idx < stride && tp >= 0 && tp < t.num_pages) return {tp, false};
    return {0, true};
}

// One row read by a load step: position j, read from page lk.pg at offset off.
void check_row(const Shape &c, const Table &t, int L, int j, Lookup lk, int off, int kbeg, int kend) {
    ++rows_checked;
    const int pg = lk.pg;
    if (pg < 0 || pg >= t.num_pages) report(c, L, "page outside the pool", j, pg);
    if (off < 0 || off >= c.P) report(c, L, "offset outside the page", j, off);
    const bool used = j >= kbeg && j < kend;
    if (lk.absent) {
        if (used) report(c, L, "used key read through an absent entry", j, pg);
        else ++fallbacks;
    }
    if (used) {
        if (j < 0 || j >= L) {
            report(c, L, "used key outside the stream", j, L);
            return;
        }
        if (pg != true_page(c, t, j)) report(c, L, "used key read from the wrong page", j, pg);
        if (off != j % c.P) report(c, L, "used key at the wrong offset", j, off);
    }
}

// Whether the non-empty intervals of iv cover [a, b) exactly once.
bool tiles_exactly(std::vector<std::pair<int, int>> iv, int a, int b) {
    std::vector<std::pair<int, int>> ne;
    for (const auto &x : iv)
        if (x.first < x.second) ne.push_back(x);
    if (!std::is_sorted(ne.begin(), ne.end())) std::sort(ne.begin(), ne.end());
    int at = a;
    for (const auto &x : ne) {
        if (x.first != at) return false;
        at = x.second;
    }
    return at == (a < b ? b : a);
}

void check_valu(const Shape &c, const CallPlan &p, const Table &t, int Ldev) {
    const int L = kernel_len(Ldev, c.max_len);
    if (Ldev > c.max_len && L != c.max_len) report(c, Ldev, "length above max_seq_len not read as max_seq_len", L, c.max_len);
    if (L <= 0) return;
    const int NB = valu_batch_keys(c.D), RPI = valu_rows_per_load(c.D);
    const int mode = valu_table_mode(c.D, c.P, p.chunk);
    const int stride = t.stride;
    const bool whole = whole_table(mode, c.ring, stride);
    int NW, NS;
    valu_load_shape(c.D, c.R * c.G, &NW, &NS);
    if (NW * NS < 16) report(c, L, "load slots do not cover a batch", NW, NS);
    if (mode == 1 && c.P < RPI) report(c, L, "per-row stepping with pages shorter than a load", c.P, RPI);
    const int lo = c.window > 0 ? std::max(0, L - c.R - c.window + 1) : 0;
    std::vector<std::pair<int, int>> cover;
    std::vector<char> written(p.n_splits, 0);
    std::vector<KeyRange> ranges(p.n_splits);
    for (int split = 0; split < p.n_splits; ++split) {
        const KeyRange k = valu_keys(L, c.R, c.window, p.n_splits, p.align, p.chunk, split);
        ranges[split] = k;
        if (k.c0 >= L) continue;
        ++wg_checked;
        written[split] = 1;
        if (k.kbeg >= k.kend) report(c, L, "written piece with no keys", k.kbeg, k.kend);
        if (k.kend - k.c0 > p.chunk) report(c, L, "piece longer than the planned chunk", k.kend - k.c0, p.chunk);
        cover.push_back({k.kbeg, k.kend});
        if (!walk_rows) continue;
        const int b_first = (k.kbeg / NB) * NB;
        const int nb = (k.kend - b_first + NB - 1) / NB;
        const int idx0 = whole ? 0 : b_first / c.P;
        const std::vector<int> ent = cached_entries(c, t, whole, idx0);
        for (int ib = 0; ib < nb; ++ib) {
            const int b = b_first + ib * NB;
            if (mode == 0) {
                const int idx = b / c.P;
                const Lookup lk = cached_page(ent, idx - idx0);
                for (int r = 0; r < NB; ++r) check_row(c, t, L, b + r, lk, b - idx * c.P + r, k.kbeg, k.kend);
            } else if (mode == 1) {
                // each lane row steps RPI rows at a time from its first slot, crossing at most
                // one page boundary per step
                for (int w = 0; w < NW; ++w)
                    for (int lrow = 0; lrow < RPI; ++lrow) {
                        const int j0 = b + w * NS * RPI + lrow;
                        int idx = j0 / c.P, off = j0 - idx * c.P;
                        for (int i = 0; i < NS; ++i) {
                            const int j = j0 + i * RPI;
                            check_row(c, t, L, j, cached_page(ent, idx - idx0), off, k.kbeg, k.kend);
                            if (idx != j / c.P || off != j % c.P) report(c, L, "row stepping lost its page", j, idx);
                            off += RPI;
                            const bool wrap = off >= c.P;
                            off = wrap ? off - c.P : off;
                            idx += wrap ? 1 : 0;
                        }
                    }
            } else {
                for (int r = 0; r < NB; ++r) {
                    const int j = b + r;
                    check_row(c, t, L, j, global_page(c, t, j / c.P), j % c.P, k.kbeg, k.kend);
                }
            }
        }
        // the fused row write of a decode: the piece that ends at the stream's length
        if (c.R == 1 && k.kend == L) {
            int idx = (L - 1) / c.P;
            if (c.ring) idx %= c.ring;
            const int pg = idx < stride ? (whole ? ent[idx] : t.e[idx]) : -1;
            if (pg != true_page(c, t, L - 1)) report(c, L, "row write to the wrong page", L - 1, pg);
        }
    }
    if (!tiles_exactly(cover, lo, L)) report(c, L, "pieces do not cover the visible keys once", lo, L);
    // the merge of each row
    for (int r = 0; r < c.R; ++r) {
        const int pos = L - c.R + r;
        if (pos < 0) continue;
        SplitSpan sp = row_splits(L, c.R, c.window, pos, p.n_splits, p.chunk, true, p.align);
        if (plant == "merge") --sp.end;
        const int lo_r = c.window > 0 ? std::max(0, pos - c.window + 1) : 0;
        if (sp.first < 0 || sp.end > p.n_splits) report(c, L, "merge span outside the splits", sp.first, sp.end);
        std::vector<std::pair<int, int>> got;
        for (int i = std::max(sp.first, 0); i < std::min(sp.end, p.n_splits); ++i) {
            if (!written[i]) report(c, L, "merge reads a split that was not written", pos, i);
            got.push_back({std::max(ranges[i].kbeg, lo_r), std::min(ranges[i].kend, pos + 1)});
        }
        if (!tiles_exactly(got, lo_r, pos + 1)) report(c, L, "merge does not hold each key of its row once", pos, lo_r);
    }
}

void check_mfma(const Shape &c, const CallPlan &p, const Table &t, int Ldev) {
    const int L = kernel_len(Ldev, c.max_len);
    if (Ldev > c.max_len && L != c.max_len) report(c, Ldev, "length above max_seq_len not read as max_seq_len", L, c.max_len);
    if (L <= 0) return;
    // (at d 128 in table mode 0 the kernel of a split call walks 32-key halves of these tiles;
    // with pages a multiple of 64 keys they read the same rows through the same pages)
    const int KT = mfma_tile_keys(c.D);
    const int mode = mfma_table_mode(c.D, c.P, p.chunk);
    const int stride = t.stride;
    const bool whole = whole_table(mode, c.ring, stride);
    const int NQ = c.R * c.G, M = 64 * p.mp.qw;
    if (p.chunk % KT != 0) report(c, L, "chunk not a whole number of tiles", p.chunk, KT);
    if (p.mp.tiles * M < NQ) report(c, L, "query tiles do not cover the vectors", p.mp.tiles, NQ);
    // the fused row write: split 0 of the tile holding a row's first query vector writes it
    const bool fused = mfma_fuses_rows(c.D, c.P, p.chunk);
    const int new0 = L - c.R, cap = c.ring * c.P;
    std::vector<int> writers(fused ? c.R : 0, 0);
    for (int tile = 0; tile < p.mp.tiles; ++tile) {
        const int v0 = tile * M;
        if (v0 >= NQ) continue;
        if (fused) {
            // `--plant put`: each tile's write starts one row late
            const int rb = (v0 + c.G - 1) / c.G + (plant == "put" ? 1 : 0);
            const int re = std::min((v0 + M + c.G - 1) / c.G, c.R);
            for (int r = rb; r < re; ++r) {
                ++writers[r];
                const int pos = new0 + r;
                if (pos < 0 || !walk_rows) continue;
                int idx = pos / c.P;
                if (c.ring) idx %= c.ring;
                const int pg = idx < stride ? t.e[idx] : -1;
                if (pg >= 0 && pg < t.num_pages && pg != true_page(c, t, pos))
                    report(c, L, "fused row write to the wrong page", pos, pg);
            }
        }
        const int r_first = v0 / c.G, r_last = (std::min(NQ, v0 + M) - 1) / c.G;
        const int p_first = L - c.R + r_first, p_last = L - c.R + r_last;
        const int lo_tile = c.window > 0 ? std::max(0, p_first - c.window + 1) : 0;
        std::vector<std::pair<int, int>> cover;
        std::vector<char> written(p.n_splits, 0);
        std::vector<KeyRange> ranges(p.n_splits);
        for (int split = 0; split < p.n_splits; ++split) {
            const KeyRange k = mfma_keys(L, c.R, c.window, p.chunk, split, p.mp.direct, r_first, r_last);
            ranges[split] = k;
            if (k.kbeg >= k.kend) continue;
            ++wg_checked;
            written[split] = 1;
            if (k.kend - k.c0 > p.chunk) report(c, L, "chunk overrun", k.kend - k.c0, p.chunk);
            cover.push_back({k.kbeg, k.kend});
            if (fused && cap > 0) {
                // keys read from the pages: [kbeg, min(kend, new0)); a written position p
                // shares the slot of key p - cap, so none of [kbeg + cap, min(kend, new0) + cap)
                // may be one of [max(new0, 0), L)
                const int64_t a0 = std::max<int64_t>((int64_t)k.kbeg + cap, std::max(new0, 0));
                const int64_t a1 = std::min<int64_t>((int64_t)std::min(k.kend, new0) + cap, L);
                if (a0 < a1) report(c, L, "a key read from the pages shares its slot with a written row", k.kbeg, a0);
            }
            if (!walk_rows) continue;
            const int kt_first = (k.kbeg / KT) * KT;
            const int nt = (k.kend - kt_first + KT - 1) / KT;
            const int idx0 = whole ? 0 : kt_first / c.P;
            const std::vector<int> ent = cached_entries(c, t, whole, idx0);
            for (int it = 0; it < nt; ++it) {
                const int tb = kt_first + it * KT;
                for (int r = 0; r < KT; ++r) {
                    const int j = tb + r;
                    if (mode == 0) {
                        const int idx = tb / c.P;
                        check_row(c, t, L, j, cached_page(ent, idx - idx0), tb - idx * c.P + r, k.kbeg, k.kend);
                    } else if (mode == 1) {
                        check_row(c, t, L, j, cached_page(ent, j / c.P - idx0), j % c.P, k.kbeg, k.kend);
                    } else {
                        check_row(c, t, L, j, global_page(c, t, j / c.P), j % c.P, k.kbeg, k.kend);
                    }
                }
            }
        }
        if (!tiles_exactly(cover, lo_tile, std::max(p_last + 1, lo_tile)))
            report(c, L, "chunks do not cover the tile's keys once", lo_tile, p_last + 1);
        if (p.mp.direct) {
            if (p.n_splits != 1) report(c, L, "direct call with several splits", p.n_splits, 1);
            continue;
        }
        for (int r = r_first; r <= r_last; ++r) {
            const int pos = L - c.R + r;
            if (pos < 0) continue;
            SplitSpan sp = row_splits(L, c.R, c.window, pos, p.n_splits, p.chunk, false, p.align);
            if (plant == "merge") --sp.end;
            const int lo_r = c.window > 0 ? std::max(0, pos - c.window + 1) : 0;
            if (sp.first < 0 || sp.end > p.n_splits) report(c, L, "merge span outside the splits", sp.first, sp.end);
            std::vector<std::pair<int, int>> got;
            for (int i = std::max(sp.first, 0); i < std::min(sp.end, p.n_splits); ++i) {
                if (!written[i]) report(c, L, "merge reads a split that was not written", pos, i);
                got.push_back({std::max(ranges[i].kbeg, lo_r), std::min(ranges[i].kend, pos + 1)});
            }
            if (!tiles_exactly(got, lo_r, pos + 1)) report(c, L, "merge does not hold each key of its row once", pos, lo_r);
        }
    }
    for (int r = 0; r < (int)writers.size(); ++r)
        if (writers[r] != 1) report(c, L, "a new row is not written exactly once", r, writers[r]);
}

void check_shape(const Shape &c, std::mt19937 &rng) {
    CallPlan p;
    if (!call_plan(c.D, c.G, c.R, c.S, c.Hkv, c.P, c.max_len, c.window, &p)) {
        report(c, 0, "no plan for a supported shape", c.R, c.G);
        return;
    }
    const int need = c.ring ? c.ring : (int)(((int64_t)c.max_len + c.P - 1) / c.P);
    const Table t = make_table(need + c.extra_stride, rng());
    std::vector<int> Ls;
    if (!walk_rows) {
        Ls = {c.R, c.max_len / 3 + 37, c.max_len - 1, c.max_len, c.max_len + 1, INT_MAX};
    } else {
        Ls = {0, 1, c.R - 1, c.R, c.R + 1, c.P - 1, c.P, c.P + 1, 2 * c.P + 3, 63, 64, 65,
              c.max_len / 2, c.max_len - 1, c.max_len, c.max_len + 1, 2 * c.max_len + 7, INT_MAX, -3};
        if (c.window > 0) {
            Ls.push_back(c.window + c.R - 1);
            Ls.push_back(c.window + c.R);
        }
        std::uniform_int_distribution<int> u(1, c.max_len);
        for (int i = 0; i < 4; ++i) Ls.push_back(u(rng));
    }
    for (int L : Ls) {
        ++lengths_checked;
        if (p.mfma) check_mfma(c, p, t, L);
        else check_valu(c, p, t, L);
    }
}

}  // namespace

int main(int argc, char **argv) {
    for (int i = 1; i + 1 < argc; ++i)
        if (!std::strcmp(argv[i], "--plant")) plant = argv[i + 1];
    std::mt19937 rng(20240611u);
    std::vector<Shape> shapes;
    const int Ds[] = {128, 256, 512};
    // (G, R) pairs of the VALU kernel (R G < 16) and of the MFMA kernel
    const int GR[][2] = {{4, 1}, {4, 2}, {4, 3}, {8, 1}, {12, 1}, {4, 4}, {4, 8}, {8, 2}, {8, 4},
                         {8, 8}, {8, 32}, {12, 2}, {12, 4}, {16, 1}, {16, 4}, {4, 128}, {8, 256}};
    const int Ps[] = {1, 3, 16, 37, 64, 100, 512};
    const int maxes[] = {700, 5920, 16000, 40960};
    const int windows[] = {0, 1, 100, 4096};
    // every combination's plan is checked; the load walk runs on a seeded sample of them
    std::uniform_real_distribution<double> coin(0.0, 1.0);
    for (int D : Ds)
        for (const auto &gr : GR)
            for (int P : Ps)
                for (int mx : maxes)
                    for (int W : windows)
                        for (int ringed = 0; ringed < 2; ++ringed) {
                            if (ringed && W == 0) continue;
                            const int R = gr[1];
                            if (mx < R) continue;
                            int ring = 0;
                            if (ringed) ring = (W + R - 1 + P - 1) / P + 1;
                            const int S = coin(rng) < 0.5 ? 1 : 12;
                            const int extra = coin(rng) < 0.5 ? 0 : 5;
                            if (coin(rng) < 0.12) shapes.push_back({D, gr[0], R, S, 8, P, mx, W, ring, extra});
                        }
    // full layers whose table is exactly the cache (160 pages), with pages that are and are not
    // a multiple of the load step, and streams up to their last position
    for (int D : Ds)
        for (const auto &gr : GR)
            for (int P : {37, 64, 100})
                shapes.push_back({D, gr[0], gr[1], 12, 8, P, 160 * P, 0, 0, 0});
    // long streams
    for (const auto &gr : GR) {
        shapes.push_back({128, gr[0], gr[1], 12, 8, 512, 262144, 0, 0, 0});
        shapes.push_back({512, gr[0], gr[1], 1, 8, 37, 65536, 4096, 0, 0});
    }
    for (const Shape &c : shapes) check_shape(c, rng);
    // the longest streams a call may describe, and the widest window: ranges and merge spans
    walk_rows = false;
    std::vector<Shape> limit;
    const int GRL[][2] = {{8, 1}, {4, 3}, {8, 4}, {16, 4}, {8, 256}};
    for (int D : Ds)
        for (const auto &gr : GRL)
            for (int P : {37, 512})
                for (int W : {0, 1, 4096, KV_MAX_SEQ_LEN - 1, KV_MAX_SEQ_LEN})
                    limit.push_back({D, gr[0], gr[1], 12, 8, P, KV_MAX_SEQ_LEN, W, 0, 0});
    for (const Shape &c : limit) check_shape(c, rng);
    shapes.insert(shapes.end(), limit.begin(), limit.end());
    if (plant == "overflow") {
        volatile int big = INT_MAX - 3;
        std::printf("planted: split_piece over %d positions\n", (int)big);
        std::printf("piece %d\n", split_piece(big, 0, 8, 64));
    }
    std::printf("shapes %zu lengths %lld workgroups %lld rows %lld absent-entry rows %lld outside-cache lookups %lld "
                "violations %lld\n",
                shapes.size(), lengths_checked, wg_checked, rows_checked, fallbacks, outside, violations);
    return violations ? 1 : 0;
}
