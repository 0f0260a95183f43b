"""Host-side tests of the C-ABI library (no GPU needed; no kernel is launched).

* The built library exports exactly the entry points include/kvpaged.h declares (an ABI
  tripwire: a new or missing export fails here).
* Bad arguments are refused with the documented status before any launch, and leave no state
  change.
* Leases and releases hand out exactly the ids the oracle's lease model predicts.
"""
import ctypes
import os
import random
import re
import subprocess

import pytest

import torch

import oracle
from paged_kv_cache_rows_amd import binding

# The refusal tests pass made-up device addresses that the checks must reject before any
# launch.  They are host-logic tests for a CPU-only machine: on a GPU host a check that wrongly
# let a case through would launch on those addresses, so they are skipped there.
host_only = pytest.mark.skipif(torch.cuda.is_available(), reason="fake device pointers; CPU-only host")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvpaged.h")
CSRC = os.path.join(ROOT, "paged_kv_cache_rows_amd", "csrc")


def _newest_source_mtime():
    paths = [HEADER] + [os.path.join(CSRC, f) for f in os.listdir(CSRC)]
    return max(os.path.getmtime(p) for p in paths)


@pytest.fixture(scope="session")
def lib():
    if not os.path.exists(binding.LIB_PATH) or os.path.getmtime(binding.LIB_PATH) < _newest_source_mtime():
        from paged_kv_cache_rows_amd import build
        build.build()
    return binding.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M))


def test_header_declares_the_six_named_entry_points():
    names = declared_functions()
    for n in ("kv_pool_create", "kv_page_lease", "kv_rows_put", "paged_attn_decode",
              "paged_attn_verify", "paged_attn_prefill"):
        assert n in names
    assert names == set(binding.EXPORTS)


def test_library_exports_exactly_the_declared_symbols(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    ours = {s for s in exported if s.startswith(("kv_", "paged_attn_"))}
    assert ours == declared_functions()
    for name in declared_functions():
        assert hasattr(lib, name)
    assert binding.abi_version() == 1


def _desc(num_pages=8, P=64, Hkv=1, D=128, streams=2, order=None):
    # Host-only calls never dereference the page pointers; any 16-byte aligned value will do.
    fo = None
    keep = None
    if order is not None:
        keep = (ctypes.c_int32 * len(order))(*order)
        fo = ctypes.cast(keep, ctypes.POINTER(ctypes.c_int32))
    d = binding.PoolDesc(num_pages, P, Hkv, D, streams, 0x10000, 0x20000, fo)
    return d, keep


def _create(lib, **kw):
    d, keep = _desc(**kw)
    h = ctypes.c_void_p()
    st = lib.kv_pool_create(ctypes.byref(d), ctypes.byref(h))
    return st, h, keep


@pytest.mark.parametrize("kw,status", [
    (dict(num_pages=0), binding.KV_E_ARG),
    (dict(P=0), binding.KV_E_ARG),
    (dict(D=12), binding.KV_E_ARG),
    (dict(streams=0), binding.KV_E_ARG),
    (dict(order=[0, 1, 2, 3, 4, 5, 6, 6]), binding.KV_E_ARG),
    (dict(order=[0, 1, 2, 3, 4, 5, 6, 8]), binding.KV_E_ARG),
])
def test_pool_create_refuses_bad_geometry(lib, kw, status):
    st, h, _ = _create(lib, **kw)
    assert st == status and not h.value
    assert lib.kv_last_error()


def test_lease_is_all_or_nothing(lib):
    st, h, _ = _create(lib, num_pages=8)
    assert st == 0
    ids = (ctypes.c_int32 * 16)()
    assert lib.kv_page_lease(h, 0, 5, ids) == 0
    assert list(ids[:5]) == [0, 1, 2, 3, 4]
    n = ctypes.c_int32()
    assert lib.kv_page_lease(h, 1, 4, ids) == binding.KV_E_NO_PAGES
    lib.kv_pool_free_count(h, ctypes.byref(n))
    assert n.value == 3
    assert lib.kv_page_lease(h, 2, 1, ids) == binding.KV_E_ARG        # stream out of range
    assert lib.kv_page_lease(h, 0, -1, ids) == binding.KV_E_ARG
    assert lib.kv_page_release(h, 0) == 0
    lib.kv_pool_free_count(h, ctypes.byref(n))
    assert n.value == 8
    lib.kv_pool_destroy(h)


@pytest.mark.parametrize("seed", range(8))
def test_leases_match_the_oracle_model(lib, seed):
    # seeds 0..3: the queue policy throughout; 4..7: the policy switches at random
    rng = random.Random(seed)
    N, S = 60, 6
    order = list(range(N))
    rng.shuffle(order)
    st, h, keep = _create(lib, num_pages=N, streams=S, order=order)
    assert st == 0
    model = oracle.LeaseModel(N, S, order)
    buf = (ctypes.c_int32 * N)()
    for _ in range(300):
        s = rng.randrange(S)
        if seed >= 4 and rng.random() < 0.05:
            pol = rng.choice(["queue", "contiguous"])
            assert lib.kv_pool_set_lease_policy(
                h, binding.KV_LEASE_CONTIGUOUS if pol == "contiguous" else binding.KV_LEASE_QUEUE) == 0
            model.set_policy(pol)
        if rng.random() < 0.65:
            n = rng.randrange(0, 15)
            st = lib.kv_page_lease(h, s, n, buf)
            try:
                want = model.lease(s, n)
                assert st == 0 and list(buf[:n]) == want
            except oracle.NoPages:
                assert st == binding.KV_E_NO_PAGES
        else:
            assert lib.kv_page_release(h, s) == 0
            model.release(s)
        cnt = ctypes.c_int32()
        lib.kv_pool_free_count(h, ctypes.byref(cnt))
        assert cnt.value == model.free_count
        got_n = ctypes.c_int32()
        assert lib.kv_stream_pages(h, s, buf, N, ctypes.byref(got_n)) == 0
        assert list(buf[:got_n.value]) == model.leased[s]
    lib.kv_pool_destroy(h)


@pytest.mark.parametrize("seed", range(4))
def test_shares_match_the_oracle_model(lib, seed):
    # leases, releases and shares (valid and refused) under both policies, library against model
    rng = random.Random(100 + seed)
    N, S = 48, 6
    st, h, keep = _create(lib, num_pages=N, streams=S)
    assert st == 0
    model = oracle.LeaseModel(N, S)
    buf = (ctypes.c_int32 * N)()
    for _ in range(300):
        s = rng.randrange(S)
        if rng.random() < 0.05:
            pol = rng.choice(["queue", "contiguous"])
            assert lib.kv_pool_set_lease_policy(
                h, binding.KV_LEASE_CONTIGUOUS if pol == "contiguous" else binding.KV_LEASE_QUEUE) == 0
            model.set_policy(pol)
        r = rng.random()
        if r < 0.45:
            n = rng.randrange(0, 8)
            st = lib.kv_page_lease(h, s, n, buf)
            try:
                want = model.lease(s, n)
            except oracle.NoPages:
                assert st == binding.KV_E_NO_PAGES
            else:
                assert st == 0 and list(buf[:n]) == want
        elif r < 0.75:
            d = rng.randrange(S)
            n = rng.randrange(0, len(model.leased[s]) + 2)
            st = lib.kv_page_share(h, s, d, n)
            try:
                model.share(s, d, n)
            except ValueError:
                assert st == binding.KV_E_ARG
            else:
                assert st == 0
        else:
            assert lib.kv_page_release(h, s) == 0
            model.release(s)
        cnt = ctypes.c_int32()
        lib.kv_pool_free_count(h, ctypes.byref(cnt))
        assert cnt.value == model.free_count
        for t in range(S):
            got_n = ctypes.c_int32()
            assert lib.kv_stream_pages(h, t, buf, N, ctypes.byref(got_n)) == 0
            assert list(buf[:got_n.value]) == model.leased[t]
    lib.kv_pool_destroy(h)


def _layout(S=1, R=1, stride=8, max_len=300, ring=0):
    # Device pointers are never dereferenced by the refusals tested here.
    return binding.Layout(S, R, 0x30000, stride, 0x40000, max_len, ring)


def _args(Hq=16, window=0, ws=0x50000, nbytes=1 << 30, scale=0.0, q=0x60000, out=0x70000):
    return binding.AttnArgs(q, out, Hq, scale, window, ws, nbytes)


@pytest.mark.parametrize("entry,lay,args,status", [
    ("paged_attn_decode", _layout(R=2), _args(), binding.KV_E_ARG),            # decode needs R == 1
    ("paged_attn_verify", _layout(R=9), _args(), binding.KV_E_ARG),            # verify is 1..8 rows
    ("paged_attn_prefill", _layout(R=0), _args(), binding.KV_E_ARG),
    ("paged_attn_decode", _layout(stride=4), _args(), binding.KV_E_ARG),       # table too short for 300/64
    ("paged_attn_decode", _layout(), _args(Hq=6), binding.KV_E_ARG),           # Hq not a multiple of Hkv = 4
    ("paged_attn_decode", _layout(), _args(Hq=12), binding.KV_E_SHAPE),        # group 3: no kernel
    ("paged_attn_decode", _layout(), _args(nbytes=16), binding.KV_E_WORKSPACE),
    ("paged_attn_decode", _layout(), _args(ws=0x50010), binding.KV_E_ARG),     # workspace misaligned
    ("paged_attn_decode", _layout(), _args(q=0x60008), binding.KV_E_ARG),      # q not 16-byte aligned
    ("paged_attn_verify", _layout(R=4), _args(out=0x70002), binding.KV_E_ARG),  # out not 16-byte aligned
    ("paged_attn_decode", _layout(), _args(window=-1), binding.KV_E_ARG),
    ("paged_attn_decode", _layout(), _args(scale=-1.0), binding.KV_E_ARG),
    ("paged_attn_decode", _layout(ring=2), _args(), binding.KV_E_ARG),         # ring without a window
    ("paged_attn_decode", _layout(ring=2), _args(window=200), binding.KV_E_ARG),  # ring 128 < window
    ("paged_attn_verify", _layout(max_len=3, R=4), _args(), binding.KV_E_ARG),   # R > max_seq_len
    ("paged_attn_decode", _layout(max_len=binding.KV_MAX_SEQ_LEN + 1, stride=(1 << 23) + 2), _args(),
     binding.KV_E_ARG),                                                        # stream past the limit
    ("paged_attn_decode", _layout(), _args(window=binding.KV_MAX_SEQ_LEN + 1), binding.KV_E_ARG),  # window past it
])
@host_only
def test_attention_refuses_before_launch(lib, entry, lay, args, status):
    d = binding.PoolDesc(8, 64, 4, 128, 2, 0x10000, 0x20000, None)
    h = ctypes.c_void_p()
    assert lib.kv_pool_create(ctypes.byref(d), ctypes.byref(h)) == 0
    st = getattr(lib, entry)(h, ctypes.byref(lay), ctypes.byref(args), None)
    assert st == status, lib.kv_last_error()
    assert lib.kv_last_error()
    lib.kv_pool_destroy(h)


def test_head_dim_without_kernel_is_a_shape_error(lib):
    d = binding.PoolDesc(8, 64, 1, 64, 2, 0x10000, 0x20000, None)
    h = ctypes.c_void_p()
    assert lib.kv_pool_create(ctypes.byref(d), ctypes.byref(h)) == 0
    n = ctypes.c_size_t()
    st = lib.paged_attn_workspace_size(h, ctypes.byref(_layout()), ctypes.byref(_args(Hq=4)), ctypes.byref(n))
    assert st == binding.KV_E_SHAPE
    lib.kv_pool_destroy(h)


def test_workspace_size_depends_on_shape_only(lib):
    d = binding.PoolDesc(100, 512, 8, 128, 12, 0x10000, 0x20000, None)
    h = ctypes.c_void_p()
    assert lib.kv_pool_create(ctypes.byref(d), ctypes.byref(h)) == 0
    n = ctypes.c_size_t()
    lay = binding.Layout(12, 1, 0x30000, 80, 0x40000, 40960, 0)
    assert lib.paged_attn_workspace_size(h, ctypes.byref(lay), ctypes.byref(_args(Hq=64)), ctypes.byref(n)) == 0
    # 12 streams x 8 KV heads = 96 (stream, head) groups and about 1536 workgroups: 16 even
    # pieces per stream; 12 streams x 64 heads x 16 x (128 + 2) floats
    assert n.value == 12 * 64 * 16 * 130 * 4
    lib.kv_pool_destroy(h)


def _splits(lib, S, R, Hkv, G, D, P, max_len, window=0):
    """Split count of an attention call, read from its workspace size."""
    d = binding.PoolDesc(100000, P, Hkv, D, S, 0x10000, 0x20000, None)
    h = ctypes.c_void_p()
    assert lib.kv_pool_create(ctypes.byref(d), ctypes.byref(h)) == 0
    lay = binding.Layout(S, R, 0x30000, (max_len + P - 1) // P, 0x40000, max_len, 0)
    n = ctypes.c_size_t()
    assert lib.paged_attn_workspace_size(h, ctypes.byref(lay), ctypes.byref(_args(Hq=Hkv * G, window=window)),
                                         ctypes.byref(n)) == 0, lib.kv_last_error()
    lib.kv_pool_destroy(h)
    per_split = S * R * Hkv * G * (D + 2) * 4
    assert n.value % per_split == 0
    return n.value // per_split


@pytest.mark.parametrize("S,R,Hkv,G,D,P,max_len,window,splits", [
    (4, 8, 8, 8, 128, 512, 9200, 0, 8),      # the verify window: 4 x 8 x 8 = 256 workgroups, one round
    (4, 8, 8, 8, 128, 512, 36800, 0, 8),     # 4096-key chunks would need 9 (288 workgroups, two rounds)
    (4, 8, 8, 8, 128, 37, 36800, 0, 8),      # the same with pages of 37 (chunks still cached)
    (12, 8, 8, 8, 128, 512, 40960, 0, 8),    # 96 groups: 768 workgroups, three whole rounds
    (12, 2, 8, 8, 128, 512, 40960, 0, 8),    # 2 rows x GQA 8 = 16 query vectors: MFMA, as above
    (1, 4, 2, 8, 512, 37, 9000, 0, 94),      # d 512: chunks of 3 tiles, 188 workgroups
    (2, 8, 8, 8, 128, 512, 3000, 100, 2),    # window of 100: its keys fit one chunk, plus the edge
    (1, 128, 8, 4, 128, 512, 40960, 0, 4),   # a 128-row prompt chunk far into its stream: 8 tiles x 8
                                             # heads x 4 chunks = 256 workgroups, one round
])
def test_verify_splits_fill_whole_rounds(lib, S, R, Hkv, G, D, P, max_len, window, splits):
    # Rows that span a small part of the keys (verify windows, late prompt chunks) give every
    # workgroup about the same work and one workgroup fills a CU, so the call runs in rounds of
    # 256 workgroups: the split count must not leave a round nearly empty.
    assert _splits(lib, S, R, Hkv, G, D, P, max_len, window) == splits


@host_only
def test_rows_put_refuses_bad_layouts(lib):
    d = binding.PoolDesc(8, 64, 1, 128, 2, 0x10000, 0x20000, None)
    h = ctypes.c_void_p()
    assert lib.kv_pool_create(ctypes.byref(d), ctypes.byref(h)) == 0
    assert lib.kv_rows_put(h, ctypes.byref(_layout(R=0)), 0x1000, 0x2000, None) == binding.KV_E_ARG
    assert lib.kv_rows_put(h, ctypes.byref(_layout()), None, 0x2000, None) == binding.KV_E_ARG
    assert lib.kv_rows_put(h, ctypes.byref(_layout()), 0x1008, 0x2000, None) == binding.KV_E_ARG   # misaligned rows
    assert lib.kv_rows_put(h, ctypes.byref(_layout()), 0x1000, 0x2004, None) == binding.KV_E_ARG
    assert lib.kv_rows_put(h, ctypes.byref(_layout(ring=1, R=65, max_len=300)), 0x1000, 0x2000, None) == binding.KV_E_ARG
    assert lib.kv_rows_put(None, ctypes.byref(_layout()), 0x1000, 0x2000, None) == binding.KV_E_ARG
    lib.kv_pool_destroy(h)


@host_only
def test_verify_tree_refuses_before_launch(lib):
    d = binding.PoolDesc(8, 64, 4, 128, 2, 0x10000, 0x20000, None)
    h = ctypes.c_void_p()
    assert lib.kv_pool_create(ctypes.byref(d), ctypes.byref(h)) == 0
    f = lib.paged_attn_verify_tree
    assert f(h, ctypes.byref(_layout(R=4)), ctypes.byref(_args()), None, None) == binding.KV_E_ARG     # no mask
    assert f(h, ctypes.byref(_layout(R=9)), ctypes.byref(_args()), 0x80000, None) == binding.KV_E_ARG  # R > 8
    assert f(h, ctypes.byref(_layout(R=4)), ctypes.byref(_args(Hq=12)), 0x80000, None) == binding.KV_E_SHAPE
    assert lib.kv_last_error()
    lib.kv_pool_destroy(h)


def test_library_follows_the_hand_worked_contiguous_sequence(lib):
    import json
    fx = json.load(open(os.path.join(ROOT, "tests", "golden", "contiguous_leases.json")))
    st, h, _ = _create(lib, num_pages=fx["num_pages"], streams=fx["max_streams"])
    assert st == 0
    buf = (ctypes.c_int32 * fx["num_pages"])()
    pol = {"queue": binding.KV_LEASE_QUEUE, "contiguous": binding.KV_LEASE_CONTIGUOUS}
    for step in fx["steps"]:
        if step["op"] == "policy":
            assert lib.kv_pool_set_lease_policy(h, pol[step["policy"]]) == 0
        elif step["op"] == "release":
            assert lib.kv_page_release(h, step["stream"]) == 0
        else:
            r = lib.kv_page_lease(h, step["stream"], step["n"], buf)
            if step["expect"] == "no_pages":
                assert r == binding.KV_E_NO_PAGES
            else:
                assert r == 0 and list(buf[:step["n"]]) == step["expect"], step
        if "free_after" in step:
            cnt = ctypes.c_int32()
            lib.kv_pool_free_count(h, ctypes.byref(cnt))
            assert cnt.value == len(step["free_after"])
    for s, want in enumerate(fx["final_leased"]):
        n = ctypes.c_int32()
        assert lib.kv_stream_pages(h, s, buf, fx["num_pages"], ctypes.byref(n)) == 0
        assert list(buf[:n.value]) == want
    assert lib.kv_pool_set_lease_policy(h, 7) == binding.KV_E_ARG
    lib.kv_pool_destroy(h)


@host_only
def test_decode_put_refuses_before_launch(lib):
    d = binding.PoolDesc(8, 64, 4, 128, 2, 0x10000, 0x20000, None)
    h = ctypes.c_void_p()
    assert lib.kv_pool_create(ctypes.byref(d), ctypes.byref(h)) == 0
    f = lib.paged_attn_decode_put
    assert f(h, ctypes.byref(_layout(R=2)), ctypes.byref(_args()), 0x90000, 0xA0000, None) == binding.KV_E_ARG
    assert f(h, ctypes.byref(_layout()), ctypes.byref(_args()), None, 0xA0000, None) == binding.KV_E_ARG
    assert f(h, ctypes.byref(_layout()), ctypes.byref(_args(Hq=12)), 0x90000, 0xA0000, None) == binding.KV_E_SHAPE
    assert f(h, ctypes.byref(_layout()), ctypes.byref(_args()), 0x90008, 0xA0000, None) == binding.KV_E_ARG   # misaligned
    assert lib.kv_last_error()
    lib.kv_pool_destroy(h)


def test_every_call_raises_without_the_library(tmp_path):
    # a copy of the package without its built library: the binding raises on the first call
    # that needs the library and never falls back to another implementation
    import shutil
    import sys
    import textwrap
    shutil.copytree(os.path.join(ROOT, "paged_kv_cache_rows_amd"), tmp_path / "paged_kv_cache_rows_amd",
                    ignore=shutil.ignore_patterns("*.so", "_build", "__pycache__"))
    code = textwrap.dedent("""
        from paged_kv_cache_rows_amd import binding
        calls = (lambda: binding.Pool(8, 64, 1, 128, 1, device="cpu"), binding.abi_version, binding.load)
        for call in calls:
            try:
                call()
            except RuntimeError as e:
                assert "is missing" in str(e), e
            else:
                raise SystemExit("a call ran without the library")
        print("all raised")
    """)
    r = subprocess.run([sys.executable, "-c", code], cwd=tmp_path, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and "all raised" in r.stdout, r.stdout + r.stderr


@host_only
def test_decode_put_static_refuses_before_launch(lib):
    d = binding.PoolDesc(8, 64, 4, 128, 2, 0x10000, 0x20000, None)
    h = ctypes.c_void_p()
    assert lib.kv_pool_create(ctypes.byref(d), ctypes.byref(h)) == 0
    f = lib.paged_attn_decode_put_static
    assert f(h, ctypes.byref(_layout(R=2)), ctypes.byref(_args()), 0x90000, 0xA0000, None) == binding.KV_E_ARG
    assert f(h, ctypes.byref(_layout()), ctypes.byref(_args()), None, 0xA0000, None) == binding.KV_E_ARG
    assert f(h, ctypes.byref(_layout()), ctypes.byref(_args(Hq=12)), 0x90000, 0xA0000, None) == binding.KV_E_SHAPE
    lib.kv_pool_destroy(h)
    # partials larger than the library's scratch: refused with KV_E_WORKSPACE before anything
    # touches a device (200 streams of 64 query heads at a 40k ceiling need about 100 MB)
    d = binding.PoolDesc(100, 512, 8, 128, 2, 0x10000, 0x20000, None)
    assert lib.kv_pool_create(ctypes.byref(d), ctypes.byref(h)) == 0
    big = binding.Layout(200, 1, 0x30000, 80, 0x40000, 40960, 0)
    n = ctypes.c_size_t()
    assert lib.paged_attn_workspace_size(h, ctypes.byref(big), ctypes.byref(_args(Hq=64)), ctypes.byref(n)) == 0
    assert n.value > binding.STATIC_SCRATCH_BYTES
    assert f(h, ctypes.byref(big), ctypes.byref(_args(Hq=64)), 0x90000, 0xA0000, None) == binding.KV_E_WORKSPACE
    assert b"scratch" in lib.kv_last_error()
    # a call that fits goes on to look up the scratch array, which needs a device: without one
    # the lookup fails and is reported, still before any launch
    small = binding.Layout(12, 1, 0x30000, 80, 0x40000, 40960, 0)
    assert lib.paged_attn_workspace_size(h, ctypes.byref(small), ctypes.byref(_args(Hq=64)), ctypes.byref(n)) == 0
    assert n.value <= binding.STATIC_SCRATCH_BYTES
    assert f(h, ctypes.byref(small), ctypes.byref(_args(Hq=64)), 0x90000, 0xA0000, None) == binding.KV_E_DEVICE
    lib.kv_pool_destroy(h)


def test_static_scratch_size_matches_the_header():
    text = open(HEADER).read()
    m = re.search(r"#define KV_STATIC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == binding.STATIC_SCRATCH_BYTES


@pytest.mark.parametrize("D,Hq,R", [(128, 16, 1), (128, 32, 4), (512, 32, 4)])
def test_the_longest_stream_and_widest_window_are_planned(lib, D, Hq, R):
    # at KV_MAX_SEQ_LEN (and a window as wide) the workspace size is computed without refusal;
    # one position more is refused
    d = binding.PoolDesc(8, 64, 4, D, 2, 0x10000, 0x20000, None)
    h = ctypes.c_void_p()
    assert lib.kv_pool_create(ctypes.byref(d), ctypes.byref(h)) == 0
    n = ctypes.c_size_t()
    top = binding.KV_MAX_SEQ_LEN
    stride = top // 64
    for window in (0, top):
        st = lib.paged_attn_workspace_size(h, ctypes.byref(_layout(R=R, stride=stride, max_len=top)),
                                           ctypes.byref(_args(Hq=Hq, window=window)), ctypes.byref(n))
        assert st == binding.KV_OK and n.value > 0, lib.kv_last_error()
    st = lib.paged_attn_workspace_size(h, ctypes.byref(_layout(R=R, stride=stride + 1, max_len=top + 1)),
                                       ctypes.byref(_args(Hq=Hq)), ctypes.byref(n))
    assert st == binding.KV_E_ARG
    lib.kv_pool_destroy(h)


def test_max_seq_len_limit_matches_the_header():
    text = open(os.path.join(ROOT, "include", "kvpaged.h")).read()
    m = re.search(r"#define KV_MAX_SEQ_LEN \(1 << (\d+)\)", text)
    assert m and 1 << int(m.group(1)) == binding.KV_MAX_SEQ_LEN
