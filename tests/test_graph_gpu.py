"""A whole decode step (plan upload + every layer's pa_decode_run) captured in
a HIP graph and replayed: every replay must equal the eager step bit for bit,
with the program's own eager work and synchronisations between replays."""
import numpy as np
import pytest
import torch

import workloads
from tests.gpu_harness import Staged, compare

pytestmark = pytest.mark.gpu


def test_graph_replays_equal_the_eager_step():
    lens = [300, 1, 4097, 64, 0, 1500, 2048, 17]
    w = workloads.custom(lens, seed=51, layers=4)
    st = Staged(w, layers=(0, 1, 2, 3))
    plan = st.pool.plan(w.ctx_lens)
    pinned = torch.from_numpy(plan.host.copy()).pin_memory()
    outs = [torch.zeros_like(st.dev[L][0]) for L in range(4)]
    rng = np.random.default_rng(1)
    knew = [torch.from_numpy(rng.standard_normal((w.batch, 8, 128)).astype(np.float16)).cuda()
            for _ in range(4)]
    vnew = [torch.from_numpy(rng.standard_normal((w.batch, 8, 128)).astype(np.float16)).cuda()
            for _ in range(4)]

    def step():
        plan.dev.copy_(pinned, non_blocking=True)
        for L in range(4):
            q, tables = st.dev[L]
            st.pool.run(L, plan, q, outs[L], tables, w.scale, k_new=knew[L], v_new=vnew[L])

    step()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    # the appended tokens are in the pool now; a read-only oracle check of layer 2
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(4):
        for o in outs:
            o.fill_(float("nan"))          # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for L in range(4):
            assert torch.equal(outs[L].view(torch.int16), eager[L].view(torch.int16)), (rep, L)
    # the appended values landed: a read-only decode of layer 2 gives the same bits
    q, tables = st.dev[2]
    again = torch.empty_like(q)
    st.pool.run(2, plan, q, again, tables, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(again.view(torch.int16), eager[2].view(torch.int16))
    st.close()


@pytest.mark.parametrize("fp8,prompt_only", [(False, False), (True, False), (False, True), (True, True)])
def test_graph_replays_of_a_mixed_step_equal_the_eager_step(fp8, prompt_only):
    """A chunked-prefill / mixed step over two layers (decode rows, whole and
    cut prompt tiles, merges; or prompt tiles alone, which take the split
    kernels) captured once and replayed: every replay gives the eager bits,
    and the eager step matches the oracle."""
    import oracle
    import paged_kv_cache_64_amd as pa

    q_lens = [40, 300, 7] if prompt_only else [1, 40, 1, 300, 7]
    hist = [0, 3000, 20] if prompt_only else [700, 0, 4095, 3000, 20]
    lens = [h + n for h, n in zip(hist, q_lens)]
    w = workloads.custom(lens, seed=52 + fp8, layers=2)
    scales = (0.1, 0.0173)
    st = Staged(w, layers=(0, 1), dtype=pa.PA_FP8_E4M3 if fp8 else pa.PA_F16, kv_scales=scales)
    starts = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    rows = int(starts[-1])
    qs = [torch.from_numpy(w.q_rows(rows, L)).cuda() for L in range(2)]
    plan = st.pool.prefill_plan(starts, lens)
    assert plan.info.num_merges > 0 and plan.info.num_prefill_items > 0
    assert (plan.info.num_items == 0) == prompt_only
    pinned = torch.from_numpy(plan.host.copy()).pin_memory()
    outs = [torch.zeros_like(q) for q in qs]

    def step():
        plan.dev.copy_(pinned, non_blocking=True)
        for L in range(2):
            st.pool.prefill_run(L, plan, qs[L], outs[L], st.dev[L][1], w.scale)

    step()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for L in range(2):
            assert torch.equal(outs[L].view(torch.int16), eager[L].view(torch.int16)), (rep, L)
    # layer 1 of the eager step against the oracle
    q, tables, ids, k, v = st.host[1]
    kc, vc, t2 = oracle.relabelled_cache(ids, k, v, tables, w.ctx_lens, 16)
    qh = w.q_rows(rows, 1)
    if fp8:
        ref = oracle.prefill_e4m3(qh, oracle.quantize_e4m3(kc, scales[0]), oracle.quantize_e4m3(vc, scales[1]),
                                  t2, starts, lens, w.scale, 16, *scales)
    else:
        ref = oracle.prefill(qh, kc, vc, t2, starts, lens, w.scale, 16)
    compare(f"graph mixed fp8={fp8} prompt_only={prompt_only}", eager[1], ref)
    st.close()
