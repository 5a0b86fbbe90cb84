"""The append + decode step captured as a HIP graph (how a serving loop, and
bench.py, run it): every replay must reproduce the eager result bit for bit,
with ordinary eager work and synchronisations between replays."""
import pytest
import torch

from mla_synth import workload

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

from gpu_harness import GpuCase  # noqa: E402


@pytest.mark.parametrize("batch,max_prefix,kv_chunk", [(5, 300, 128), (40, 400, 64)], ids=["grid", "work_list"])
def test_graph_replay_matches_eager(batch, max_prefix, kv_chunk):
    """kv_chunk 64 over 40 ragged sequences launches the attention from the
    device-built work list, which every replay rebuilds."""
    wl = workload("dsv2_ragged_paged_256", name=f"graph_b{batch}", batch=batch, max_prefix=max_prefix)
    print(f"[graph] case {wl.name} B={wl.batch}", flush=True)
    case = GpuCase(wl)
    mla = case.mla
    s = wl.shape
    Tq = case.q.shape[0]
    ws = torch.empty(mla.mla_decode_workspace_bytes(case.layer, wl.batch, Tq, case.max_q_len,
                                                    case.max_seq_len, kv_chunk), dtype=torch.uint8, device="cuda")
    aws = torch.empty(max(1, mla.mla_append_workspace_bytes(case.layer, Tq)), dtype=torch.uint8, device="cuda")

    def step(out, stream=None):
        mla.mla_append_latent(case.layer, case.x_new_dev, case.cu_q, case.prefix_dev, case.page_table, case.cache,
                              workspace=aws, stream=stream)
        mla.mla_decode(case.layer, case.q_dev, case.cu_q, case.seq_lens, case.page_table, case.cache, out,
                       case.max_q_len, case.max_seq_len, kv_chunk=kv_chunk, workspace=ws, stream=stream)

    eager = torch.empty((Tq, s.H, s.d_v), dtype=case.dt, device="cuda")
    step(eager)
    torch.cuda.synchronize()

    out_g = torch.empty_like(eager)
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            step(out_g)
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()

    other = torch.empty_like(eager)
    for rep in range(3):
        out_g.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, eager), f"graph replay {rep} differs from the eager result"
        step(other)                     # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(other, eager)
    print("[graph] 3 replays identical to eager", flush=True)


def test_two_stream_graph_matches_eager():
    """The step as bench.py times it: the append on a side stream beside the
    absorb phase (they touch disjoint data), the attention and output after
    both; captured with a fork/join pair of events and replayed."""
    wl = workload("dsv2_ragged_paged_256", name="graph2", batch=5, max_prefix=300)
    print(f"[graph] case {wl.name} B={wl.batch}, two streams", flush=True)
    case = GpuCase(wl)
    mla = case.mla
    s = wl.shape
    Tq = case.q.shape[0]
    ws = torch.empty(mla.mla_decode_workspace_bytes(case.layer, wl.batch, Tq, case.max_q_len,
                                                    case.max_seq_len, 128), dtype=torch.uint8, device="cuda")
    aws = torch.empty(max(1, mla.mla_append_workspace_bytes(case.layer, Tq)), dtype=torch.uint8, device="cuda")
    dec = (case.layer, case.q_dev, case.cu_q, case.seq_lens, case.page_table, case.cache)

    eager = torch.empty((Tq, s.H, s.d_v), dtype=case.dt, device="cuda")
    mla.mla_append_latent(case.layer, case.x_new_dev, case.cu_q, case.prefix_dev, case.page_table, case.cache,
                          workspace=aws)
    mla.mla_decode(*dec, eager, case.max_q_len, case.max_seq_len, kv_chunk=128, workspace=ws)
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    fork, join = torch.cuda.Event(), torch.cuda.Event()

    def step(out):
        main = torch.cuda.current_stream()
        fork.record(main)
        side.wait_event(fork)
        mla.mla_append_latent(case.layer, case.x_new_dev, case.cu_q, case.prefix_dev, case.page_table, case.cache,
                              workspace=aws, stream=side)
        join.record(side)
        mla.mla_decode_phases(*dec, out, case.max_q_len, case.max_seq_len, kv_chunk=128, workspace=ws,
                              phases=mla.MLA_PHASE_ABSORB)
        main.wait_event(join)
        mla.mla_decode_phases(*dec, out, case.max_q_len, case.max_seq_len, kv_chunk=128, workspace=ws,
                              phases=mla.MLA_PHASE_ATTEND | mla.MLA_PHASE_OUTPUT)

    out_g = torch.empty_like(eager)
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            step(out_g)
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()

    for rep in range(3):
        out_g.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, eager), f"two-stream graph replay {rep} differs from the eager result"
        other = torch.empty_like(eager)
        mla.mla_decode(*dec, other, case.max_q_len, case.max_seq_len, kv_chunk=128, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(other, eager)
    print("[graph] 3 two-stream replays identical to eager", flush=True)


def test_decode_step_graph_replay_matches_eager():
    """mla_decode_step (the query absorb and the append finish in one launch)
    captured as a graph: three replays, with eager steps between them, each
    bit-identical to the eager call."""
    wl = workload("dsv2_ragged_paged_256", name="graph_step", batch=4, max_prefix=250)
    print(f"[graph] case {wl.name} B={wl.batch}", flush=True)
    case = GpuCase(wl)
    mla = case.mla
    s = wl.shape
    Tq = case.q.shape[0]
    ws = torch.empty(mla.mla_decode_step_workspace_bytes(case.layer, wl.batch, Tq, Tq, case.max_q_len,
                                                         case.max_seq_len), dtype=torch.uint8, device="cuda")

    def step(out):
        mla.mla_decode_step(case.layer, case.x_new_dev, case.cu_q, case.prefix_dev, case.q_dev, case.cu_q,
                            case.seq_lens, case.page_table, case.cache, out, case.max_q_len, case.max_seq_len,
                            workspace=ws)

    eager = torch.empty((Tq, s.H, s.d_v), dtype=case.dt, device="cuda")
    step(eager)
    torch.cuda.synchronize()
    out_g = torch.empty_like(eager)
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            step(out_g)
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    other = torch.empty_like(eager)
    for rep in range(3):
        out_g.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, eager), f"decode step graph replay {rep} differs from the eager result"
        step(other)
        torch.cuda.synchronize()
        assert torch.equal(other, eager)
    print("[graph] decode step: 3 replays identical to eager", flush=True)
