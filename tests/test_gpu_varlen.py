"""GPU parity of continuous batching over a state pool: ragged sequences
(prefills of several lengths, one-token decode steps, an empty sequence)
packed back to back in one call, each on its own slot of the conv and SSM
pools (some starting fresh), against the fp64 oracle's batched entry on the
same pools; elementwise at 2e-2, conv pool bit for bit, unused slots
untouched. Invalid offsets or slots are refused on the device: nothing is
written and the status reports it."""
import numpy as np
import pytest

from gpu_util import TOL, check, dev, host
from mamba_ssd_selective_mixer_amd import synth
from oracle import oracle

pytestmark = pytest.mark.gpu
VARLEN = -12


@pytest.fixture(scope="module")
def ops():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mamba_ssd_selective_mixer_amd import ops as _ops
    return _ops


def batch_case(ops, cfg, lens, slots, has, S, with_bias=False, check_ref=True, slow=False):
    import torch
    bf = torch.bfloat16
    T = int(sum(lens))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    prm = synth.layer_params(cfg, slow_decay=slow, with_bias=with_bias)
    inp = synth.prefill_inputs(cfg, batch=1, seqlen=T)
    r = np.random.default_rng(cfg.index + 77)
    cpool = synth.to_io(np.sqrt(0.1) * r.standard_normal((S, cfg.conv_width - 1, cfg.channels)),
                        cfg.dtype)
    spool = (np.sqrt(0.1) * r.standard_normal((S, cfg.nheads, cfg.headdim, cfg.dstate))
             ).astype(np.float32)
    d = ops.SSDDims(len(lens), T, cfg.nheads, cfg.headdim, cfg.ngroups, cfg.dstate,
                    cfg.conv_width, cfg.chunk, bf)
    gc, gs = dev(cpool, bf), dev(spool)
    ws = ops.workspace(ops.ssd_mixer_varlen_workspace_bytes(d, S))
    out = torch.full((T, cfg.hp), 7.0, dtype=bf, device="cuda")
    hs = None if has is None else torch.tensor(has, dtype=torch.uint8, device="cuda")
    ops.ssd_mixer_varlen(d, torch.tensor(cu, device="cuda"),
                         torch.tensor(slots, dtype=torch.int32, device="cuda"),
                         dev(inp["xbc"][0], bf), dev(inp["z"][0], bf), dev(inp["dt"][0], bf),
                         dev(prm["A"]), dev(prm["D"]), dev(prm["conv_w"], bf),
                         dev(prm["conv_b"], bf), dev(prm["norm_w"], bf), gc, gs,
                         eps=prm["eps"], has_state=hs, out=out, ws=ws)
    rc = ops.ssd_workspace_status(ws)
    res = (host(out), host(gc), host(gs), rc, cpool, spool)
    if not check_ref:
        return res
    assert rc == 0
    ro, rc_, rs = oracle.mixer_varlen(cu, slots, has, inp["xbc"][0], inp["z"][0], inp["dt"][0],
                                      prm["A"], prm["D"], prm["conv_w"], prm["conv_b"],
                                      prm["norm_w"], prm["eps"], cfg.nheads, cfg.headdim,
                                      cfg.ngroups, cfg.dstate, cpool, spool)
    check("varlen out", res[0], ro, TOL["bf16"])
    assert np.array_equal(res[1], rc_), "conv pool"
    check("varlen ssm pool", res[2], rs, TOL["bf16"])
    return res


@pytest.mark.parametrize("kw", [dict(), dict(nheads=64, ngroups=2), dict(nheads=64)])
def test_mixed_prefill_and_decode(ops, kw):
    """Prefills of 300, 129, 64 and 2 tokens, three one-token decode steps
    and an empty sequence, on shuffled slots of a pool of 11 (two sequences
    fresh); norm within one block, across 8 blocks, and across 2 blocks."""
    cfg = synth.replace(synth.CONFIGS["tiny_layer"], **kw)
    lens = [300, 1, 129, 0, 2, 1, 64, 1]
    slots = [7, 0, 3, 9, 10, 5, 1, 4]
    has = [1, 1, 0, 1, 1, 0, 1, 1]
    batch_case(ops, cfg, lens, slots, has, S=11)


@pytest.mark.parametrize("kw", [dict(), dict(nheads=64)])
def test_mixed_batch_bias_slow_decay(ops, kw):
    """Conv bias and slow decay in a ragged batch: the chunk kernels carry
    each sequence's state split into S' + a bbar^T (the carried-in slot
    state split by projection), per-chunk rows in the ragged chunk table;
    prefills of 600, 257 and 2 tokens beside decode steps and an empty
    sequence, some slots fresh."""
    cfg = synth.replace(synth.CONFIGS["tiny_layer"], **kw)
    lens = [600, 1, 257, 0, 2, 1]
    slots = [4, 0, 2, 5, 1, 3]
    has = [1, 1, 0, 1, 1, 0]
    batch_case(ops, cfg, lens, slots, has, S=6, with_bias=True, slow=True)


def test_decode_only_batch(ops):
    """64 one-token sequences on a pool of 96 (a decode step of the serving
    engine through the batched entry), large-layer head count."""
    cfg = synth.replace(synth.CONFIGS["decode_loop"], chunk=128)
    r = np.random.default_rng(5)
    slots = r.permutation(96)[:64].tolist()
    batch_case(ops, cfg, [1] * 64, slots, None, S=96)


@pytest.mark.parametrize("kw,with_bias", [(dict(), False), (dict(), True),
                                          (dict(nheads=64), True)])
def test_single_sequence_matches_prefill_entry(ops, kw, with_bias):
    """One sequence through the batched entry gives the dense prefill entry's
    output and states bit for bit (same kernels, same chunks); with a conv
    bias the state split's per-chunk rows sit at the ragged chunk indices."""
    import torch
    bf = torch.bfloat16
    cfg = synth.replace(synth.CONFIGS["tiny_layer"], batch=1, seqlen=700, **kw)
    out, gc, gs, rc, cpool, spool = batch_case(ops, cfg, [700], [2], [1], S=3,
                                               with_bias=with_bias)
    prm = synth.layer_params(cfg, with_bias=with_bias)
    inp = synth.prefill_inputs(cfg, batch=1, seqlen=700)
    d = ops.SSDDims(1, 700, cfg.nheads, cfg.headdim, cfg.ngroups, cfg.dstate, 4, 128, bf)
    cs, ss = dev(cpool[2:3], bf), dev(spool[2:3])
    cb = dev(prm["conv_b"], bf) if with_bias else None
    o = ops.ssd_mixer_prefill(d, dev(inp["xbc"], bf), dev(inp["z"], bf), dev(inp["dt"], bf),
                              dev(prm["A"]), dev(prm["D"]), dev(prm["conv_w"], bf), cb,
                              dev(prm["norm_w"], bf), prm["eps"], cs, cs, ss, ss)
    assert np.array_equal(host(o)[0], out)
    assert np.array_equal(host(ss)[0], gs[2]) and np.array_equal(host(cs)[0], gc[2])


@pytest.mark.parametrize("fresh", [False, True])
def test_one_token_sequences_match_decode_entry(ops, fresh):
    """One-token sequences of a ragged batch are decode steps: beside a
    prefill, they give the decode entry's output and new states bit for bit
    (the same decode kernel, token rows and slots taken from the batch),
    resuming from their slots or starting fresh (zero states)."""
    import torch
    bf = torch.bfloat16
    cfg = synth.replace(synth.CONFIGS["tiny_layer"], chunk=128)
    lens, slots = [1, 200, 1], [4, 0, 2]
    has = [0 if fresh else 1, 1, 0 if fresh else 1]
    out, gc, gs, rc, cpool, spool = batch_case(ops, cfg, lens, slots, has, S=5)
    T = sum(lens)
    prm = synth.layer_params(cfg)
    inp = synth.prefill_inputs(cfg, batch=1, seqlen=T)
    rows = [0, 201]  # token rows of the two one-token sequences
    d = ops.SSDDims(2, 1, cfg.nheads, cfg.headdim, cfg.ngroups, cfg.dstate, 4, 128, bf)
    cs = dev(cpool[[4, 2]], bf)
    ss = dev(spool[[4, 2]])
    if fresh:
        cs.zero_()
        ss.zero_()
    y = ops.ssd_decode_step(d, dev(inp["xbc"][0][rows], bf), dev(inp["z"][0][rows], bf),
                            dev(inp["dt"][0][rows], bf), dev(prm["A"]), dev(prm["D"]),
                            dev(prm["conv_w"], bf), None, dev(prm["norm_w"], bf), prm["eps"],
                            cs, ss)
    assert np.array_equal(host(y), out[rows])
    assert np.array_equal(host(cs), gc[[4, 2]]) and np.array_equal(host(ss), gs[[4, 2]])


@pytest.mark.parametrize("lens,slots,S", [
    ([5, 3], [1, 1], 4),      # one slot used twice
    ([5, 3], [0, 4], 4),      # slot past the pool
    ([5, 3], [-1, 2], 4),     # negative slot
])
def test_invalid_slots_refused(ops, lens, slots, S):
    cfg = synth.replace(synth.CONFIGS["tiny_layer"])
    out, gc, gs, rc, cpool, spool = batch_case(ops, cfg, lens, slots, None, S=S,
                                                check_ref=False)
    assert rc == VARLEN
    assert np.all(out == 7.0), "nothing may be written"
    assert np.array_equal(gc, cpool) and np.array_equal(gs, spool)


def test_invalid_offsets_refused(ops):
    """cu_seqlens that do not end at the call's token count, or decrease."""
    import torch
    bf = torch.bfloat16
    cfg = synth.CONFIGS["tiny_layer"]
    T, S = 12, 4
    d = ops.SSDDims(2, T, cfg.nheads, cfg.headdim, cfg.ngroups, cfg.dstate, 4, 128, bf)
    prm = synth.layer_params(cfg)
    inp = synth.prefill_inputs(cfg, batch=1, seqlen=T)
    gc = torch.zeros(S, 3, cfg.channels, dtype=bf, device="cuda")
    gs = torch.zeros(S, cfg.nheads, cfg.headdim, cfg.dstate, device="cuda")
    for cu in ([0, 5, 11], [0, 7, 5], [1, 5, 12]):
        ws = ops.workspace(ops.ssd_mixer_varlen_workspace_bytes(d, S))
        out = torch.full((T, cfg.hp), 7.0, dtype=bf, device="cuda")
        ops.ssd_mixer_varlen(d, torch.tensor(cu, dtype=torch.int32, device="cuda"),
                             torch.tensor([0, 1], dtype=torch.int32, device="cuda"),
                             dev(inp["xbc"][0], bf), dev(inp["z"][0], bf), dev(inp["dt"][0], bf),
                             dev(prm["A"]), dev(prm["D"]), dev(prm["conv_w"], bf), None,
                             dev(prm["norm_w"], bf), gc, gs, out=out, ws=ws)
        assert ops.ssd_workspace_status(ws) == VARLEN, cu
        assert float(out.float().sub(7.0).abs().max()) == 0.0
        assert float(gs.abs().max()) == 0.0 and float(gc.float().abs().max()) == 0.0


def test_graph_replay_and_stream_order(ops):
    """A ragged batch (prefills and one-token decode steps) captured into a
    HIP graph replays to the eager result bit for bit on every replay, with
    the pools restored and the workspace scribbled over by eager work
    between replays (the chunk table, decode list and norm tickets are
    rebuilt by kernels, not memsets); and work the caller enqueues after the
    call on its stream sees every output and state (read back without any
    device-wide sync)."""
    import torch
    bf = torch.bfloat16
    cfg = synth.replace(synth.CONFIGS["tiny_layer"], nheads=64, chunk=128)
    lens, slots = [1, 300, 1, 1, 129, 1], [6, 0, 2, 5, 3, 1]
    T = int(sum(lens))
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32), device="cuda")
    sl = torch.tensor(slots, dtype=torch.int32, device="cuda")
    prm = synth.layer_params(cfg)
    inp = synth.prefill_inputs(cfg, batch=1, seqlen=T)
    r = np.random.default_rng(3)
    S = 7
    cpool = dev(synth.to_io(np.sqrt(0.1) * r.standard_normal((S, 3, cfg.channels)), "bf16"), bf)
    spool = dev((np.sqrt(0.1) * r.standard_normal((S, cfg.nheads, cfg.headdim, cfg.dstate))
                 ).astype(np.float32))
    d = ops.SSDDims(len(lens), T, cfg.nheads, cfg.headdim, cfg.ngroups, cfg.dstate, 4, 128, bf)
    args = (dev(inp["xbc"][0], bf), dev(inp["z"][0], bf), dev(inp["dt"][0], bf), dev(prm["A"]),
            dev(prm["D"]), dev(prm["conv_w"], bf), None, dev(prm["norm_w"], bf))
    ws = ops.workspace(ops.ssd_mixer_varlen_workspace_bytes(d, S))
    out = torch.empty(T, cfg.hp, dtype=bf, device="cuda")
    gc, gs = cpool.clone(), spool.clone()

    def call():
        ops.ssd_mixer_varlen(d, cu, sl, *args, gc, gs, eps=prm["eps"], out=out, ws=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
        # stream order: copies enqueued after the call on the same stream
        ref = (out.clone(), gc.clone(), gs.clone())
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref = tuple(host(t) for t in ref)
    assert np.array_equal(host(out), ref[0]) and np.array_equal(host(gs), ref[2])
    gc.copy_(cpool)
    gs.copy_(spool)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for i in range(3):
        gc.copy_(cpool)
        gs.copy_(spool)
        out.fill_(float("nan"))
        ws.fill_(7)
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(out), ref[0]), f"replay {i}: out"
        assert np.array_equal(host(gc), ref[1]), f"replay {i}: conv pool"
        assert np.array_equal(host(gs), ref[2]), f"replay {i}: ssm pool"
