/*
 * kvpaged.h -- C ABI of a paged KV cache and attention over it, for MI355X (gfx950).
 *
 * The operation (TensorFold PR #1620, paged K/V for Kolibri-1's full layers, opening
 * description): the full layers keep K and V in fixed-size pages of one shared pool (512
 * positions per page; the kernel-contract bullet also runs pages of 37 and 64), every stream
 * leases pages as it grows, new rows are copied into their page slots (the Writes bullet), and
 * attention reads keys through a per-stream page table passed in the call's stream order (the
 * Reads bullet); sliding layers keep ring buffers instead.  Decode and drafted verify read
 * through the table, with verify windows of 1..8 causal rows (TensorFold PR #2730, What this
 * changes: the pending token and up to seven drafts), and prompts have their own paged kernels.
 *
 * Conventions shared by every call:
 *   - Every call returns kv_status.  Nothing aborts, throws or synchronises the device.  On a
 *     non-OK status no state changed and no kernel was launched (except KV_E_DEVICE, which
 *     reports a failed launch); kv_last_error() gives the text, per calling thread.
 *   - All device buffers (pages, queries, outputs, new rows, tables, lengths, workspace) are
 *     allocated and owned by the caller and must outlive the calls that use them.  The library
 *     owns only host metadata (the pool's free list, per-stream lease lists and the number of
 *     streams holding each page) and allocates no device memory.  The one piece of device
 *     memory it holds is the fixed scratch array of paged_attn_decode_put_static, part of its
 *     code object on every GPU it runs on.
 *   - `hip_stream` is a hipStream_t (NULL = the legacy default stream).  Device work is
 *     enqueued on it asynchronously, in the order of the calls.
 *   - bf16 is the format of the high 16 bits of an IEEE binary32 (raw uint16 storage); outputs
 *     are rounded to it to nearest even.
 *   - Table contents and device lengths are trusted on the hot path; with the environment
 *     variable KVP_CHECK=1 every call copies them to the host first (synchronously) and refuses
 *     bad ones with KV_E_ARG.  Without it, a page id outside [0, num_pages) is never
 *     dereferenced (attention reads page 0 in its place; row writes skip it) and a length
 *     above max_seq_len is read as max_seq_len, so a bad table or length gives a wrong result
 *     but touches no memory outside the pool, the table and the workspace.
 */
#ifndef KVPAGED_H
#define KVPAGED_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVPAGED_ABI_VERSION 1

/* The longest stream a call may describe (kv_layout.max_seq_len) and the widest sliding window
 * (kv_attn_args.window): 2^29 positions.  Within them every position, key range, chunk end and
 * piece length the kernels and the planning form stays below 2^31 in 32-bit ints; a larger
 * value is refused with KV_E_ARG. */
#define KV_MAX_SEQ_LEN (1 << 29)

typedef enum kv_status {
    KV_OK = 0,
    KV_E_ARG = -1,        /* a null pointer, a negative or inconsistent size, a bad stream id */
    KV_E_SHAPE = -2,      /* a shape the library has no kernel for (head_dim, GQA group, rows) */
    KV_E_NO_PAGES = -3,   /* a lease asked for more pages than are free (nothing was leased) */
    KV_E_WORKSPACE = -4,  /* the workspace passed is smaller than paged_attn_workspace_size() */
    KV_E_DEVICE = -5      /* the HIP runtime reported an error for a launch */
} kv_status;

/* Opaque pool handle: host metadata only (geometry, free list, leases). */
typedef struct kv_pool kv_pool;

/* Pool geometry and storage.  K and V pages are caller-owned device arrays of bf16 laid out
 * [num_pages][num_kv_heads][page_size][head_dim]: one KV head's rows inside a page are
 * contiguous, and a row is head_dim contiguous values. */
typedef struct kv_pool_desc {
    int32_t num_pages;       /* > 0 */
    int32_t page_size;       /* P >= 1 positions per page (512 by default; any value works) */
    int32_t num_kv_heads;    /* Hkv >= 1 */
    int32_t head_dim;        /* D >= 8, a multiple of 8 (attention needs 128, 256 or 512) */
    int32_t max_streams;     /* number of stream ids [0, max_streams) that may lease */
    void *k_pages;           /* device, bf16 [num_pages][Hkv][P][D] */
    void *v_pages;           /* device, bf16 [num_pages][Hkv][P][D] */
    const int32_t *free_order; /* host, optional [num_pages]: a permutation of the page ids
                                  giving the order pages are handed out; NULL = 0,1,2,...
                                  Copied at creation. */
} kv_pool_desc;

/* One call's streams.  Stream i of the call uses row i of the page table and seq_len[i]. */
typedef struct kv_layout {
    int32_t num_streams;       /* S >= 1 */
    int32_t rows;              /* R >= 1: new rows (kv_rows_put) or query rows per stream */
    const int32_t *page_table; /* device int32 [S][table_stride]: entry i is the physical page
                                  of the stream's logical page i (full layers) or ring slot i
                                  (ring layers) */
    int32_t table_stride;      /* >= the entries a stream uses (ceil(L/P), or ring_pages) */
    const int32_t *seq_len;    /* device int32 [S]: the stream's length L >= 0 after this call's
                                  rows; the call's rows sit at positions L-R .. L-1, and rows at
                                  negative positions (R > L) are not written and see no key */
    int32_t max_seq_len;       /* host: an upper bound of seq_len over the call (sizes grids and
                                  the workspace), rows <= max_seq_len <= KV_MAX_SEQ_LEN.  A
                                  larger device length is a caller error: the
                                  kernels read it as max_seq_len, so every access stays inside
                                  the table and workspace planned for the call, and KVP_CHECK=1
                                  refuses it before launch */
    int32_t ring_pages;        /* 0: full layer, position j lives in page table[j / P];
                                  n > 0: ring of n pages, position j lives in
                                  table[(j / P) % n], so only the newest n*P positions exist */
} kv_layout;

/* Attention arguments. */
typedef struct kv_attn_args {
    const void *q;           /* device bf16 [S][R][Hq][D], 16-byte aligned */
    void *out;               /* device bf16 [S][R][Hq][D], 16-byte aligned, written in full */
    int32_t num_q_heads;     /* Hq, a multiple of Hkv; query head h reads KV head h / (Hq/Hkv) */
    float scale;             /* score scale; 0 means 1/sqrt(D) */
    int32_t window;          /* 0: full causal; W > 0: row at position p sees keys p-W+1 .. p
                                (W <= KV_MAX_SEQ_LEN) */
    void *workspace;         /* device scratch, >= paged_attn_workspace_size() bytes, 256-byte
                                aligned; its contents on entry do not matter */
    size_t workspace_bytes;
} kv_attn_args;

/* Create a pool over caller-owned pages (TensorFold PR #1620, opening description: the pool
 * is an arena planned for the streams and leased out; here the arena is the caller's pair of
 * page arrays and the leasing is below).
 * Errors: KV_E_ARG for a null desc/out/page pointer, a non-positive size, D not a multiple of
 * 8, or a free_order that is not a permutation of [0, num_pages). */
kv_status kv_pool_create(const kv_pool_desc *desc, kv_pool **out);

/* Destroy the host metadata (never the caller's pages).  NULL is accepted.  (The pool is the
 * arena of TensorFold PR #1620's opening description; its memory stays the caller's, as the
 * buffers of the launcher on the metrale glm5next_dsa select.rs page are its caller's.) */
kv_status kv_pool_destroy(kv_pool *pool);

/* Lease n pages to a stream as it grows (TensorFold PR #1620, opening description: streams
 * take pages from the shared pool as their caches grow).  Which ids are handed out follows the
 * pool's lease policy (below; by default the front of the free queue, in queue order).  They
 * are appended to the stream's lease list and written to page_ids_out (host [n]).
 * All or nothing: with fewer than n free pages it returns KV_E_NO_PAGES and changes nothing.
 * KV_E_ARG for a bad stream id, n < 0, or a null output with n > 0.  Thread-safe per pool. */
kv_status kv_page_lease(kv_pool *pool, int32_t stream, int32_t n, int32_t *page_ids_out);

/* Lease policies.
 * KV_LEASE_QUEUE (the default): the first n ids of the free queue, in queue order.
 * KV_LEASE_CONTIGUOUS: keep each stream in runs of adjacent page ids while the pool has room,
 *   and fall back to scattered pages when it does not (TensorFold PR #1620, first review, which
 *   suggests one unbroken run of pages per full layer while the pool has space to spare).  The ids come from
 *   the first of these steps that applies:
 *   1. the stream holds pages, its last leased id is t, and t+1 .. t+n are all free: those;
 *   2. the longest run of adjacent free ids that holds n (the lowest such run on a tie), say
 *      [a, b): ids start .. start+n-1 with start = a when a == 0, else a + (b - a - n) / 2
 *      (half the run's spare room stays behind the page before it, whose stream may grow);
 *   3. the n lowest free ids, in increasing order.
 * Either policy removes the ids it hands out from the free queue; releases append to its back
 * as always.  The page table is the only thing the kernels read, so the policy changes where
 * pages live, never a result.  KV_E_ARG for an unknown policy.  Thread-safe per pool. */
enum { KV_LEASE_QUEUE = 0, KV_LEASE_CONTIGUOUS = 1 };
kv_status kv_pool_set_lease_policy(kv_pool *pool, int32_t policy);

/* Give up all of a stream's pages (released pages are handed out again by later leases, which
 * the PR's model test covers).  Each page loses one holder; the pages that no other stream
 * holds (see kv_page_share) go to the back of the free queue, in the order the stream leased
 * them.  KV_E_ARG for a bad stream id.  The pages' contents are left as they are. */
kv_status kv_page_release(kv_pool *pool, int32_t stream);

/* Share a prefix of one stream's pages with another (TensorFold PR #1620, opening description,
 * Kept states bullet: a kept state is resumed and its pages reused; sharing is the form of that
 * which copies nothing).  dst_stream, which must hold no pages, takes the first n pages of
 * src_stream's lease list, in that order; each gains a holder and none leaves the free queue.
 * Later leases append to dst_stream's list as usual, and a page returns to the free queue only
 * when its last holder releases it.  Both streams' tables then point at the same pages for the
 * shared prefix, and a row written into a shared page is seen by every holder: share only pages
 * that no holder writes again (the full pages of a common prefix) and give a partly filled last
 * page its own copy (kv_page_lease + kv_pages_copy).  Errors: KV_E_ARG for bad stream ids,
 * src_stream == dst_stream, n outside [0, pages src_stream holds], or a dst_stream that holds
 * pages.  Thread-safe per pool. */
kv_status kv_page_share(kv_pool *pool, int32_t src_stream, int32_t dst_stream, int32_t n);

/* Number of free pages. */
kv_status kv_pool_free_count(const kv_pool *pool, int32_t *out);

/* Copy up to `cap` of a stream's leased page ids, in lease order, to ids_out (host); *n_out
 * receives the stream's total count (which may exceed cap). */
kv_status kv_stream_pages(const kv_pool *pool, int32_t stream, int32_t *ids_out, int32_t cap,
                          int32_t *n_out);

/* Write each stream's R new K and V rows into their page slots (TensorFold PR #1620, opening
 * description, Writes bullet: the K/V rows a layer produces are copied into the pages).
 * k_new, v_new: device bf16 [S][R][Hkv][D], 16-byte aligned.  Row r of stream s goes to
 * position seq_len[s] - R + r, i.e. page table[s][pos / P] (or ring slot (pos / P) % ring_pages)
 * at slot pos % P, for every KV head.  Rows at negative positions are skipped.  Every other
 * byte of the pool is left untouched.  Errors: KV_E_ARG (null or misaligned pointers, bad
 * sizes). */
kv_status kv_rows_put(const kv_pool *pool, const kv_layout *lay, const void *k_new,
                      const void *v_new, void *hip_stream);

/* Copy whole pages, K and V, every KV head: page dst_ids[i] receives the contents of page
 * src_ids[i] for i < n (TensorFold PR #1620, opening description, Kept states bullet: a
 * stream's state is kept by copying the pages its table walks).  Keeping a state: lease fresh
 * pages, copy the stream's table entries onto them, and the new ids form a table that reads
 * back the same cache; resuming is attending (and writing) through that table.
 * src_ids, dst_ids: device int32 [n], caller-owned.  No page may be a destination twice or be
 * both a source and a destination (the pairs run concurrently); ids outside [0, num_pages)
 * are skipped.  With KVP_CHECK=1 the ids are copied to the host first and both rules are
 * checked (KV_E_ARG).  Errors: KV_E_ARG (null pointers, n < 0). */
kv_status kv_pages_copy(const kv_pool *pool, const int32_t *src_ids, const int32_t *dst_ids, int32_t n,
                        void *hip_stream);

/* Bytes of workspace that a decode/verify/prefill call with these arguments needs: a function
 * of the call's shape only (S, R, Hkv, Hq, D, max_seq_len, window), never of the device
 * lengths or the table.  The convention is that of the metrale glm5next_dsa select.rs page
 * (module invariants and the scratch `fits` check: scratch is sized from the launch geometry
 * ahead of time, and a pass that needs more than was allocated is an error, not an overrun): every attention call checks its workspace
 * against this size before any launch and returns KV_E_WORKSPACE when it is smaller.  It holds the split partials (D + 2 floats per query vector and
 * split).  A call whose query tiles fill the GPU by themselves uses one split and writes its
 * output directly; it still asks for, and is checked against, this size. */
kv_status paged_attn_workspace_size(const kv_pool *pool, const kv_layout *lay,
                                    const kv_attn_args *a, size_t *bytes);

/* Paged GQA attention for one decode row per stream (R == 1) (TensorFold PR #1620, opening
 * description, Reads bullet: decode reads its keys through the page table).  For each stream s and
 * query head h: out = softmax(scale * q K^T) V over the keys the row sees (all positions
 * 0..L-1, or the newest `window`), K and V read through the stream's page table; a row
 * that sees no key (a stream of length 0) gets zeros.  Computed
 * with fp32 accumulation; the output is rounded to bf16 (nearest even).  Results depend only
 * on the logical cache, never on which physical pages hold it (bit for bit).
 * Errors: KV_E_ARG (R != 1, null or misaligned pointers, Hq not a multiple of Hkv), KV_E_SHAPE (no kernel
 * for this head_dim or group), KV_E_WORKSPACE (too small). */
kv_status paged_attn_decode(const kv_pool *pool, const kv_layout *lay, const kv_attn_args *a,
                            void *hip_stream);

/* kv_rows_put of one new row per stream followed by paged_attn_decode (TensorFold PR #1620,
 * opening description, Writes and Reads bullets: a layer's new K/V row is copied into the
 * pages, then attention reads through the table), in one launch where the group has fewer than
 * 16 query heads (the VALU kernel writes the row itself) or, with 16, at head_dim 128 over
 * pages of a multiple of 64 positions (as paged_attn_prefill_put), else as a row-write launch
 * followed by the attention on the same stream.  k_new, v_new: device
 * bf16 [S][1][Hkv][D] (16-byte aligned), written at position seq_len[s] - 1 exactly as
 * kv_rows_put writes it; the output and every byte of the pool afterwards equal those of the
 * two calls.  Errors as for decode, with KV_E_ARG for a null or misaligned k_new or v_new. */
kv_status paged_attn_decode_put(const kv_pool *pool, const kv_layout *lay, const kv_attn_args *a,
                                const void *k_new, const void *v_new, void *hip_stream);

/* paged_attn_decode_put for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  The split partials go to a
 * scratch array of KV_STATIC_SCRATCH_BYTES that the library keeps in the memory of each GPU it
 * runs on (from the first call on that GPU until the process ends); a->workspace and
 * a->workspace_bytes are ignored, and nothing is allocated or freed.  The caller still passes
 * every input and output.  All calls on one GPU share that GPU's array: calls that may run at
 * the same time on one GPU (on different streams, or from different threads) race on it and
 * must be ordered by the caller.  Nothing in the array needs to start at zero (every partial a
 * call reads is written earlier in the same call).  Errors as for paged_attn_decode_put, and
 * KV_E_WORKSPACE when the call needs more scratch than the array holds (the size
 * paged_attn_workspace_size reports for the same arguments must not exceed
 * KV_STATIC_SCRATCH_BYTES), KV_E_DEVICE if the array's address cannot be looked up. */
#define KV_STATIC_SCRATCH_BYTES (32u << 20)
kv_status paged_attn_decode_put_static(const kv_pool *pool, const kv_layout *lay, const kv_attn_args *a,
                                       const void *k_new, const void *v_new, void *hip_stream);

/* The same for a speculative verify window of 1 <= R <= 8 causal rows per stream (TensorFold
 * PR #2730, What this changes: the pending token plus up to seven drafts, and the window
 * kernels accept any row count).  Row r sits at position L-R+r and sees keys up to and including itself.
 * Errors as for decode, with KV_E_ARG for R outside 1..8. */
kv_status paged_attn_verify(const kv_pool *pool, const kv_layout *lay, const kv_attn_args *a,
                            void *hip_stream);

/* The same for a verify window whose R (1..8) rows are a flattened draft tree rather than a
 * chain (TensorFold PR #1620, opening description, Reads bullet: decode and drafted verify go
 * through tree attention).  tree_mask: device uint32 [S][R], caller-owned; bit i of
 * tree_mask[s][r] says that row r of stream s sees window slot i (position L-R+i): its
 * ancestors and, normally, itself.  The tree must list parents before children; bits above r
 * are ignored.  Every row sees all keys before the window (inside its sliding window, if any).
 * A row that sees no key gets zeros.  With tree_mask[s][r] = 2^(r+1) - 1 the result is
 * paged_attn_verify's, byte for byte.  Errors as for verify, with KV_E_ARG for a null mask. */
kv_status paged_attn_verify_tree(const kv_pool *pool, const kv_layout *lay, const kv_attn_args *a,
                                 const uint32_t *tree_mask, void *hip_stream);

/* The same for a prompt chunk of any R >= 1 causal rows per stream (TensorFold PR #1620,
 * opening description, Reads bullet: prompts have paged prompt kernels of their own).  A prompt is
 * processed chunk by chunk: kv_rows_put the chunk's rows, then this call with R = chunk rows.
 * Errors as for decode, with KV_E_ARG for R < 1. */
kv_status paged_attn_prefill(const kv_pool *pool, const kv_layout *lay, const kv_attn_args *a,
                             void *hip_stream);

/* kv_rows_put of a prompt chunk's R rows followed by paged_attn_prefill (TensorFold PR #1620,
 * opening description, Writes and Reads bullets), in one launch where the call runs the MFMA
 * kernel that loads whole 64-key tiles straight into LDS (R times the group at least 16,
 * head_dim 128, pages of a multiple of 64 positions, and a workgroup's keys within the 160
 * table entries it caches: every prompt chunk of up to about 10,000 keys over pages of 64, or
 * 80,000 over pages of 512), or where R = 1 on the VALU kernel; otherwise as a row-write
 * launch followed by the attention on the same stream.  In the one-launch form each
 * new row is written into its page slot by one workgroup, and the attention reads the call's
 * own rows from k_new and v_new rather than from those slots.  k_new, v_new: device bf16
 * [S][R][Hkv][D] (16-byte aligned, caller-owned), row r of stream s written at position
 * seq_len[s] - R + r exactly as kv_rows_put writes it (rows before position 0, or whose table
 * entry is out of range, are skipped).  With every new row's table entry in range, the
 * output and every byte of the pool afterwards equal those of the two calls.  A ring layer
 * needs room for window + R - 1 positions, as for the two calls.  Errors as for prefill, with
 * KV_E_ARG for a null or misaligned k_new or v_new. */
kv_status paged_attn_prefill_put(const kv_pool *pool, const kv_layout *lay, const kv_attn_args *a,
                                 const void *k_new, const void *v_new, void *hip_stream);

/* Measurement hook: when both are non-NULL, every later attention call made by this thread
 * records hipEvent_t `start` on its stream just before its part kernel (the one that streams K
 * and V) and `stop` just after it, so the caller can time that kernel alone with
 * hipEventElapsedTime.  NULL, NULL turns it off.  The events are the caller's. */
kv_status kv_set_part_events(void *start_event, void *stop_event);

/* Text of the calling thread's last non-OK status ("" if none): the reason a call was refused
 * before any launch (as the plan and scratch checks on the metrale glm5next_dsa select.rs page
 * fail with a message rather than launching). */
const char *kv_last_error(void);

/* KVPAGED_ABI_VERSION of the built library. */
int32_t kv_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KVPAGED_H */
