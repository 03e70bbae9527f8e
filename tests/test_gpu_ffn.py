"""GPU parity for q8_0_moe_ffn, the routed expert FFN, stage by stage.

A quantized mid is not unique: the GPU evaluates SwiGLU in fp32 and the
oracle in double, and a value next to a rounding tie may quantize to either
neighbour.  As the pages do for their own MoE kernels (the down stage is
judged against a CPU re-quantization of the GPU's own mid), each stage is
checked for what is unique and the rest for validity:
  mid   : GPU fp32 against the oracle's SwiGLU of the oracle's gate/up, within
          a tolerance carried through silu's derivative from the matmul bound;
  mid_q : the oracle quantizer applied to the GPU's mid, byte for byte;
  y     : the oracle's down projection of the GPU's mid_q, within tolerance;
  out   : the oracle's weighted combine of the GPU's y, within tolerance.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.helpers import assert_close, cpu_u8, oracle_quantize, say

pytestmark = pytest.mark.gpu

REL, ABS = 1e-5, 1e-6


def _q8():
    import q8_quantized_matmul_amd as q8
    return q8


def _mid_tolerance(gate, up, gate_mag, up_mag, mid_ref, clamp):
    """|mid_gpu - mid_ref| bound: the gate/up matmul bounds carried through
    d(silu(g) u)/dg and /du, plus 8 fp32 ulps of the result for the fp32
    evaluation of exp, the division and the products."""
    g = gate.astype(np.float64)
    u = up.astype(np.float64)
    if clamp > 0:
        g = np.minimum(g, clamp)
        u = np.clip(u, -clamp, clamp)
    sig = 1.0 / (1.0 + np.exp(-g))
    dsilu = sig * (1.0 + g * (1.0 - sig))
    tg = REL * gate_mag + ABS
    tu = REL * up_mag + ABS
    return np.abs(dsilu * u) * tg + np.abs(g * sig) * tu + 8 * 2.0 ** -24 * np.abs(mid_ref) + 1e-30


def _build(n_expert, d_model, d_ff, tag):
    q8 = _q8()
    mats, mats_o = {}, {}
    for which, (rows, cols) in (("gate", (d_ff, d_model)), ("up", (d_ff, d_model)),
                                ("down", (d_model, d_ff))):
        st = torch.empty((n_expert, rows, q8.row_bytes(cols)), dtype=torch.uint8, device="cuda")
        lst = []
        for e in range(n_expert):
            w = workloads.normal((rows, cols), 0.02, "cuda", "ffn", tag, which, e)
            q8.q8_0_quantize_act(w, out=st[e])
            lst.append(oracle_quantize(w))
        torch.cuda.synchronize()
        for e in range(n_expert):
            assert np.array_equal(cpu_u8(st[e]), lst[e]), f"{which}[{e}] quantization differs"
        mats[which], mats_o[which] = st, lst
    return mats, mats_o


def _run(mats, n_expert, d_model, d_ff, sel, weights, x, clamp):
    q8 = _q8()
    n_tok, n_used = sel.shape
    pairs = n_tok * n_used
    xq = q8.q8_0_quantize_act(x)
    mid = torch.full((pairs, d_ff), float("nan"), device="cuda")
    mid_q = torch.full((pairs, q8.row_bytes(d_ff)), 0xAB, dtype=torch.uint8, device="cuda")
    y = torch.full((pairs, d_model), float("nan"), device="cuda")
    out = torch.full((n_tok, d_model), float("nan"), device="cuda")
    _, ws = q8.q8_0_moe_ffn(q8.expert_table(mats["gate"]), q8.expert_table(mats["up"]),
                            q8.expert_table(mats["down"]), n_expert, sel.cuda(), weights.cuda(),
                            xq, d_model, d_ff, clamp, out=out, mid=mid, mid_q=mid_q, y=y)
    torch.cuda.synchronize()
    return xq, mid, mid_q, y, out, ws


def _check(mats_o, d_model, d_ff, sel, weights, x, xq, mid, mid_q, y, out, clamp, where,
           tokens=None):
    """Stage checks on the given tokens (all by default)."""
    sel = sel.numpy()
    n_tok, n_used = sel.shape
    toks = np.arange(n_tok) if tokens is None else np.asarray(tokens)
    xq_o = oracle_quantize(x[torch.as_tensor(toks, device=x.device)])
    assert np.array_equal(cpu_u8(xq)[toks], xq_o), f"{where}: x_q differs"
    s = sel[toks]
    gate, gmag, bad = oracle.moe_grouped(mats_o["gate"], s, xq_o, d_model, d_ff, 0)
    up, umag, _ = oracle.moe_grouped(mats_o["up"], s, xq_o, d_model, d_ff, 0)
    valid = (s >= 0) & (s < len(mats_o["gate"]))
    mid_ref = oracle.swiglu(gate, up, clamp)
    prow = (toks[:, None] * n_used + np.arange(n_used)[None, :])  # pair rows of these tokens
    m = mid.cpu().numpy()[prow]
    tol = _mid_tolerance(gate, up, gmag, umag, mid_ref, clamp)
    err = np.abs(m.astype(np.float64) - mid_ref)
    assert np.all(err[valid] <= tol[valid]), f"{where}: mid outside tolerance, worst {np.max(err[valid] / tol[valid]):.3g}"
    # mid_q is the quantization of the GPU's own mid.
    mq = cpu_u8(mid_q)[prow.reshape(-1)].reshape(len(toks), n_used, -1)
    for t in range(len(toks)):
        for j in range(n_used):
            if valid[t, j]:
                assert np.array_equal(mq[t, j], oracle.quantize(m[t, j][None, :])[0]), \
                    f"{where}: mid_q of pair ({toks[t]}, {j}) is not the quantization of mid"
    # y is the down projection of the GPU's mid_q.
    yr, ymag, _ = oracle.moe_grouped(mats_o["down"], s, mq.reshape(len(toks) * n_used, -1), d_ff,
                                     d_model, 1)
    yg = y.cpu().numpy()[prow]
    assert np.all(np.isnan(yg[~valid])), f"{where}: invalid pairs must have NaN y"
    assert_close(yg[valid], yr[valid], ymag[valid], f"{where} y")
    # out is the weighted combine of the GPU's y.
    o_ref, omag = oracle.moe_combine(yg, weights.numpy()[toks])
    assert_close(out.cpu().numpy()[toks], o_ref, omag, f"{where} out")
    return int((~valid).sum())


def _routing(n_expert, n_tok, n_used, seed):
    g = torch.Generator().manual_seed(seed)
    sel = torch.stack([torch.randperm(n_expert, generator=g)[:n_used] for _ in range(n_tok)])
    w = torch.rand((n_tok, n_used), generator=g)
    return sel.to(torch.int32), w.to(torch.float32)


@pytest.mark.parametrize("d_model,d_ff,n_expert,n_tok,n_used,clamp", [
    (256, 128, 6, 5, 3, 0.0), (256, 128, 6, 5, 3, 10.0), (512, 256, 9, 11, 4, 0.0),
    (4096, 2048, 12, 6, 8, 10.0), (1024, 4096, 5, 3, 2, 0.0),
    (64, 64, 1, 1, 1, 0.0), (128, 64, 3, 2, 3, 10.0), (16384, 2048, 4, 3, 2, 0.0)])
def test_moe_ffn_small(d_model, d_ff, n_expert, n_tok, n_used, clamp):
    q8 = _q8()
    tag = f"{d_model}_{d_ff}_{n_expert}"
    mats, mats_o = _build(n_expert, d_model, d_ff, tag)
    sel, w = _routing(n_expert, n_tok, n_used, d_model + n_tok)
    x = workloads.normal((n_tok, d_model), 1.0, "cuda", "ffn", tag, "x")
    say(f"[ffn] d_model={d_model} d_ff={d_ff} E={n_expert} T={n_tok} k={n_used} clamp={clamp}")
    xq, mid, mid_q, y, out, ws = _run(mats, n_expert, d_model, d_ff, sel, w, x, clamp)
    assert q8.moe_invalid_count(ws) == 0
    _check(mats_o, d_model, d_ff, sel, w, x, xq, mid, mid_q, y, out, clamp, "ffn small")
    # Deterministic: a second call gives the same bits.
    _, _, _, y2, out2, _ = _run(mats, n_expert, d_model, d_ff, sel, w, x, clamp)
    assert torch.equal(out.view(torch.int32), out2.view(torch.int32))
    assert torch.equal(y.view(torch.int32), y2.view(torch.int32))


def _random_ffn(n_cases, seed):
    """Seeded FFN calls over the widths the call accepts (64 ... 4096 values a
    row, and 8192/16384 for d_model), 1-20 experts, 1-40 tokens, with and
    without the clamp; the oracle's work per case is bounded."""
    rng = np.random.default_rng(seed)
    widths = [64 * 2 ** i for i in range(7)]
    cases = []
    while len(cases) < n_cases:
        d_model = int(rng.choice(widths + [8192, 16384]))
        d_ff = int(rng.choice(widths + [8192]))
        n_expert = int(rng.integers(1, 21))
        n_used = int(rng.integers(1, min(8, n_expert) + 1))
        n_tok = int(rng.choice([1, 2, 5, 16, 17, 40]))
        clamp = float(rng.choice([0.0, 10.0]))
        if 3 * n_tok * n_used * d_model * d_ff <= 1.2e8 and n_expert * d_model * d_ff <= 2e8:
            cases.append((d_model, d_ff, n_expert, n_tok, n_used, clamp))
    return cases


@pytest.mark.parametrize("d_model,d_ff,n_expert,n_tok,n_used,clamp", _random_ffn(8, 11))
def test_moe_ffn_random_shapes(d_model, d_ff, n_expert, n_tok, n_used, clamp):
    q8 = _q8()
    tag = f"r{d_model}_{d_ff}_{n_expert}"
    mats, mats_o = _build(n_expert, d_model, d_ff, tag)
    sel, w = _routing(n_expert, n_tok, n_used, d_ff + n_tok)
    x = workloads.normal((n_tok, d_model), 1.0, "cuda", "ffn", tag, "x")
    say(f"[ffn random] d_model={d_model} d_ff={d_ff} E={n_expert} T={n_tok} k={n_used} clamp={clamp}")
    xq, mid, mid_q, y, out, ws = _run(mats, n_expert, d_model, d_ff, sel, w, x, clamp)
    assert q8.moe_invalid_count(ws) == 0
    _check(mats_o, d_model, d_ff, sel, w, x, xq, mid, mid_q, y, out, clamp, "ffn random")


def test_moe_ffn_clamp_is_active():
    # Large activations push gate and up past the limit: the clamped and
    # unclamped results differ, and each matches its own oracle.
    d_model, d_ff, n_expert, n_tok, n_used = 256, 128, 4, 4, 2
    mats, mats_o = _build(n_expert, d_model, d_ff, "clamp")
    sel, w = _routing(n_expert, n_tok, n_used, 5)
    x = workloads.normal((n_tok, d_model), 1.0, "cuda", "ffn", "clamp", "x") * 400.0
    res = {}
    for clamp in (0.0, 10.0):
        xq, mid, mid_q, y, out, _ = _run(mats, n_expert, d_model, d_ff, sel, w, x, clamp)
        _check(mats_o, d_model, d_ff, sel, w, x, xq, mid, mid_q, y, out, clamp, f"clamp {clamp}")
        res[clamp] = mid.cpu().numpy()
    assert np.abs(res[0.0]).max() > 10.0 and not np.array_equal(res[0.0], res[10.0])


def test_moe_ffn_invalid_ids_and_duplicates():
    q8 = _q8()
    d_model, d_ff, n_expert, n_tok, n_used = 512, 256, 6, 7, 3
    mats, mats_o = _build(n_expert, d_model, d_ff, "inv")
    sel, w = _routing(n_expert, n_tok, n_used, 7)
    sel[1, 2] = 6          # out of range
    sel[4, 0] = -3         # out of range
    sel[5, 1] = sel[5, 0]  # duplicate id in one token's list
    x = workloads.normal((n_tok, d_model), 1.0, "cuda", "ffn", "inv", "x")
    xq, mid, mid_q, y, out, ws = _run(mats, n_expert, d_model, d_ff, sel, w, x, 0.0)
    assert q8.moe_invalid_count(ws) == 2
    bad = _check(mats_o, d_model, d_ff, sel, w, x, xq, mid, mid_q, y, out, 0.0, "ffn invalid")
    assert bad == 2
    o = out.cpu().numpy()
    assert np.all(np.isnan(o[1])) and np.all(np.isnan(o[4]))
    assert not np.isnan(np.delete(o, [1, 4], axis=0)).any()


def test_moe_ffn_workload_sampled():
    """The MoE workload at full size (256 experts, 64 tokens x 8 slots); the
    oracle checks every stage of 3 sampled tokens (24 pairs) in full."""
    q8 = _q8()
    cfg = workloads.MOE
    E, k, T, D, F = cfg["n_expert"], cfg["n_used"], cfg["n_tok"], cfg["d_model"], cfg["d_ff"]
    sel = workloads.moe_routing()
    g = torch.Generator().manual_seed(23)
    w = torch.rand((T, k), generator=g)
    x, _ = workloads.moe_acts("cuda")
    say("[ffn] quantizing 256 experts x 3")
    stacks = {}
    for which, (rows, cols) in (("gate", (F, D)), ("up", (F, D)), ("down", (D, F))):
        st = torch.empty((E, rows, q8.row_bytes(cols)), dtype=torch.uint8, device="cuda")
        for e in range(E):
            q8.q8_0_quantize_act(workloads.moe_expert(e, which, "cuda"), out=st[e])
        stacks[which] = st
    xq, mid, mid_q, y, out, ws = _run(stacks, E, D, F, sel, w, x, 0.0)
    assert q8.moe_invalid_count(ws) == 0
    toks = [3, 31, 62]
    used = sorted({int(e) for e in sel[toks].reshape(-1)})
    # Oracle weights only for the experts these tokens use (others never read).
    mats_o = {}
    for which in ("gate", "up", "down"):
        lst = [None] * E
        for e in used:
            lst[e] = oracle_quantize(workloads.moe_expert(e, which, "cuda"))
            assert np.array_equal(cpu_u8(stacks[which][e]), lst[e])
        empty = np.zeros_like(lst[used[0]])
        mats_o[which] = [m if m is not None else empty for m in lst]
    say(f"[ffn] oracle on tokens {toks}")
    _check(mats_o, D, F, sel, w, x, xq, mid, mid_q, y, out, 0.0, "ffn workload", tokens=toks)


def test_moe_ffn_graph_replay_matches_eager():
    """The call is capturable (no host sync, no memset): replays equal the
    eager result bit for bit, with eager work on the same buffers between."""
    q8 = _q8()
    d_model, d_ff, n_expert, n_tok, n_used = 512, 256, 6, 5, 3
    mats, _ = _build(n_expert, d_model, d_ff, "graph")
    sel, w = _routing(n_expert, n_tok, n_used, 9)
    x = workloads.normal((n_tok, d_model), 1.0, "cuda", "ffn", "graph", "x")
    xq = q8.q8_0_quantize_act(x)
    tables = [q8.expert_table(mats[k]) for k in ("gate", "up", "down")]
    sel_d, w_d = sel.cuda(), w.cuda()
    out = torch.empty((n_tok, d_model), device="cuda")
    ws = torch.empty(q8.q8_0_moe_ffn_workspace_bytes(n_tok, n_used, n_expert, d_model, d_ff),
                     dtype=torch.uint8, device="cuda")
    call = lambda: q8.q8_0_moe_ffn(*tables, n_expert, sel_d, w_d, xq, d_model, d_ff, 0.0,
                                   out=out, workspace=ws)
    call()
    torch.cuda.synchronize()
    eager = out.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            call()
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        out.fill_(float("nan"))
        ws.fill_(0x5A)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), eager.view(torch.int32)), f"replay {rep} differs"
        assert q8.moe_invalid_count(ws) == 0
