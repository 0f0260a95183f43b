"""GPU tests of calls captured in HIP graphs (a decode step replayed while the streams grow,
verify windows and prompt chunks replayed over fixed inputs) and of calls on side streams.

The launch grid of a call is sized from the host ceiling `max_seq_len` and every stream length
is read from device memory, so one captured step (kv_rows_put of each stream's new row, then
paged_attn_decode) stays valid for later lengths up to that ceiling, as long as the pool and the
page tables stay where they are.  (TensorFold PR #1620, opening description: attaching the paged
caches drops any step graph captured before them; here the pages never move, so a captured step
only needs the leases to cover the growth.)

Every replay is compared byte for byte with the same step run eagerly, and with the oracle;
eager work (updating the lengths, the new rows and the queries) runs between the replays.
"""
import pytest
import torch

from gpu_support import assert_close, new_cache, oracle_for, oracle_from_history, poisoned_workspace, say
from paged_kv_cache_rows_amd import binding, staging, workloads

pytestmark = pytest.mark.gpu

STEPS = 4


def _w():
    # final lengths; the history before the replayed steps is STEPS rows shorter
    return workloads.Workload(name="graph", streams=3, kv_heads=2, group=8, head_dim=128, page_size=64,
                              rows=1, lengths=[900, 403, 1500], spare_frac=0.2, min_spares=2, seed=21)


def _rows(hist, lengths, dev):
    """The row each stream writes at position length - 1, as [S][1][Hkv][D]."""
    return torch.stack([hist[s][L - 1:L] for s, L in enumerate(lengths)]).to(dev).contiguous()


def test_captured_decode_step_replays_as_streams_grow():
    w = _w()
    c, _, _ = new_cache(w, history=False)
    ks, vs = workloads.kv_history(w)
    start = [L - STEPS for L in w.lengths]
    staging.write_history(c, ks, vs, upto=start)
    dev = c.table.device
    max_len = max(w.lengths)

    # static inputs and outputs of the captured step
    seq = torch.tensor(start, dtype=torch.int32, device=dev)
    k_new = _rows(ks, start, dev)
    v_new = _rows(vs, start, dev)
    q = workloads.normal_bf16((w.streams, 1, w.q_heads, w.head_dim), 500).to(dev)
    out = torch.empty_like(q)
    ws = torch.empty(binding.workspace_size(c.pool, c.table, seq, 1, w.q_heads, max_len), dtype=torch.uint8,
                     device=dev)

    def step(o):
        binding.rows_put(c.pool, c.table, seq, k_new, v_new, max_len)
        binding.decode(c.pool, q, c.table, seq, max_len, out=o, workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(out)                       # warm-up: rewrites row start - 1 with its own values
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(out)
    torch.cuda.synchronize()

    for i in range(STEPS):
        lengths = [L0 + i + 1 for L0 in start]
        say(f"replay {i}: lengths {lengths}")
        seq.copy_(torch.tensor(lengths, dtype=torch.int32))
        k_new.copy_(_rows(ks, lengths, dev))
        v_new.copy_(_rows(vs, lengths, dev))
        q.copy_(workloads.normal_bf16(q.shape, 501 + i))
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        eager = torch.empty_like(q)
        step(eager)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), eager.view(torch.int16)), f"replay {i} differs from eager"
        assert_close(got, oracle_from_history(ks, vs, q, lengths), f"replay {i}")
    del g


@pytest.mark.parametrize("entry,R,G,D,Hkv", [("verify", 8, 8, 128, 2), ("verify", 3, 4, 128, 2),
                                              ("verify", 4, 8, 512, 1), ("prefill", 64, 4, 128, 2),
                                              ("prefill", 512, 4, 128, 8)])
def test_captured_verify_and_prompt_calls_replay_byte_equal(entry, R, G, D, Hkv):
    # a verify window (VALU at 3 rows x GQA 4, MFMA split with its merge otherwise) or a prompt
    # chunk (split plan at 64 rows, direct plan at 512) captured once; before every replay the
    # output and the workspace are refilled with NaN bytes by eager work
    w = workloads.Workload(name="graph", streams=2, kv_heads=Hkv, group=G, head_dim=D, page_size=64,
                           rows=R, lengths=[1500, 700], spare_frac=0.2, min_spares=2, seed=41)
    say(f"captured {entry} R={R} G={G} D={D}")
    c, _, _ = new_cache(w)
    q = workloads.queries(w).cuda()
    ws = poisoned_workspace(c, R, w.q_heads)
    fn = {"verify": binding.verify, "prefill": binding.prefill}[entry]
    eager = fn(c.pool, q, c.table, c.seq_len, c.max_seq_len, workspace=ws)
    torch.cuda.synchronize()
    out = torch.empty_like(q)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn(c.pool, q, c.table, c.seq_len, c.max_seq_len, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn(c.pool, q, c.table, c.seq_len, c.max_seq_len, out=out, workspace=ws)
    for i in range(STEPS):
        out.view(torch.int16).fill_(0x7FC0)
        ws.fill_(0xFF)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {i} differs from eager"
    assert_close(out, oracle_for(c, q), f"captured {entry} R={R} D={D}")


def test_calls_on_two_streams_at_once_match_the_default_stream():
    # a verify window (MFMA split and merge) and a decode (VALU) on two side streams, enqueued
    # in turn with no synchronisation between them: the library keeps no device state of its
    # own (every buffer is the caller's), so each equals the same call on the default stream
    wa = workloads.Workload(name="sa", streams=2, kv_heads=2, group=8, head_dim=128, page_size=64,
                            rows=8, lengths=[1500, 700], spare_frac=0.2, min_spares=2, seed=51)
    wb = workloads.Workload(name="sb", streams=3, kv_heads=2, group=8, head_dim=128, page_size=37,
                            rows=1, lengths=[900, 40, 2000], spare_frac=0.2, min_spares=2, seed=52)
    say("verify and decode on two side streams")
    ca, _, _ = new_cache(wa)
    cb, _, _ = new_cache(wb)
    qa = workloads.queries(wa).cuda()
    qb = workloads.queries(wb).cuda()
    ref_a = binding.verify(ca.pool, qa, ca.table, ca.seq_len, ca.max_seq_len)
    ref_b = binding.decode(cb.pool, qb, cb.table, cb.seq_len, cb.max_seq_len)
    wsa = poisoned_workspace(ca, wa.rows, wa.q_heads)
    wsb = poisoned_workspace(cb, wb.rows, wb.q_heads)
    oa, ob = torch.empty_like(qa), torch.empty_like(qb)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        with torch.cuda.stream(s1):
            binding.verify(ca.pool, qa, ca.table, ca.seq_len, ca.max_seq_len, out=oa, workspace=wsa)
        with torch.cuda.stream(s2):
            binding.decode(cb.pool, qb, cb.table, cb.seq_len, cb.max_seq_len, out=ob, workspace=wsb)
    torch.cuda.synchronize()
    assert torch.equal(oa.view(torch.int16), ref_a.view(torch.int16))
    assert torch.equal(ob.view(torch.int16), ref_b.view(torch.int16))


def test_calls_given_a_stream_allocate_their_buffers_on_it():
    # no out and no workspace passed: the binding allocates both for the call, on the stream the
    # kernels run on; meanwhile the default stream allocates, fills and frees buffers of the
    # same sizes, which must never land in memory a side-stream call is still using
    w = workloads.Workload(name="sa", streams=2, kv_heads=2, group=8, head_dim=128, page_size=64,
                           rows=8, lengths=[3000, 1700], spare_frac=0.2, min_spares=2, seed=55)
    c, _, _ = new_cache(w)
    q = workloads.queries(w).cuda()
    ref = binding.verify(c.pool, q, c.table, c.seq_len, c.max_seq_len)
    torch.cuda.synchronize()
    nbytes = binding.workspace_size(c.pool, c.table, c.seq_len, w.rows, w.q_heads, c.max_seq_len)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(20):
        outs.append(binding.verify(c.pool, q, c.table, c.seq_len, c.max_seq_len, stream=side))
        junk = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda")
        junk2 = torch.full_like(q.view(torch.int16), 0x7FC0)
        del junk, junk2
    torch.cuda.synchronize()
    for o in outs:
        assert torch.equal(o.view(torch.int16), ref.view(torch.int16))
    assert_close(ref, oracle_for(c, q), "verify on a side stream")
