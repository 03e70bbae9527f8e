"""GPU parity for q8_0_matmul_list, the multi-projection call.

Every item of every call is checked three ways:
  * the x_q bytes it writes equal the oracle quantizer's (bit-exact);
  * its fp32 output is within the stated tolerance of the oracle;
  * its output is bit-identical to separate q8_0_quantize_act + q8_0_matmul
    calls without workspace: a merged launch may not change any result.
Weights are quantized on the GPU (they are data to the kernels) and, for the
oracle side, by the oracle; the two are compared byte for byte.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.helpers import assert_close, cpu_u8, oracle_quantize, say

pytestmark = pytest.mark.gpu


def _q8():
    import q8_quantized_matmul_amd as q8
    return q8


def _weights(w):
    q8 = _q8()
    wq = q8.q8_0_quantize_act(w.cuda().contiguous())
    torch.cuda.synchronize()
    wq_o = oracle_quantize(w)
    assert np.array_equal(cpu_u8(wq), wq_o), "weight quantization differs"
    return wq, wq_o


def _run(specs, n_tok, tag):
    """specs: dicts with in_dim, out_dim, mode in {"x", "x+xq", "xq"} and
    optionally share=j (use item j's fp32 x) or w/x tensors."""
    q8 = _q8()
    items, keep = [], []
    for i, sp in enumerate(specs):
        k, n = sp["in_dim"], sp["out_dim"]
        w = sp.get("w")
        if w is None:
            w = workloads.normal((n, k), 0.02, "cuda", "list", tag, i, "w")
        if "share" in sp:
            x = keep[sp["share"]]["x"]
        else:
            x = sp.get("x")
            if x is None:
                x = workloads.normal((n_tok, k), 1.0, "cuda", "list", tag, i, "x")
        x = x.cuda().contiguous()
        wq, wq_o = _weights(w)
        out = torch.full((n_tok, n), float("nan"), device="cuda")
        xq = None
        if "xq" in sp["mode"]:
            xq = torch.full((n_tok, q8.row_bytes(k)), 0xAB, dtype=torch.uint8, device="cuda")
            if sp["mode"] == "xq":
                q8.q8_0_quantize_act(x, out=xq)
        it = dict(out=out, w=wq, in_dim=k, out_dim=n)
        if "x" in sp["mode"].split("+"):
            it["x"] = x
        if xq is not None:
            it["x_q"] = xq
        items.append(it)
        keep.append(dict(x=x, wq=wq, wq_o=wq_o, xq=xq, out=out, k=k, n=n, mode=sp["mode"]))
    say(f"[list] {tag}: n_tok={n_tok} items={[(s['in_dim'], s['out_dim'], s['mode']) for s in specs]}")
    q8.q8_0_matmul_list(items, n_tok)
    torch.cuda.synchronize()
    for i, kp in enumerate(keep):
        where = f"{tag}[{i}] in={kp['k']} out={kp['n']} {kp['mode']}"
        xq_o = oracle_quantize(kp["x"])
        if kp["xq"] is not None:
            assert np.array_equal(cpu_u8(kp["xq"]), xq_o), f"{where}: x_q bytes differ"
        ref, mag, _ = oracle.matmul(kp["wq_o"], xq_o, kp["k"])
        assert_close(kp["out"].cpu().numpy(), ref, mag, where)
        sep_xq = q8.q8_0_quantize_act(kp["x"])
        sep = q8.q8_0_matmul(kp["wq"], sep_xq, kp["k"], kp["n"], n_tok,
                             workspace=torch.empty(1, dtype=torch.uint8, device="cuda"))
        torch.cuda.synchronize()
        assert torch.equal(kp["out"].view(torch.int32), sep.view(torch.int32)), \
            f"{where}: differs from separate calls"
    return keep


def test_list_decode5_projections():
    """The five decode projections of one layer in one call, fp32 inputs."""
    specs = [dict(in_dim=p["in_dim"], out_dim=p["out_dim"], mode="x+xq", w=p["w"], x=p["x"])
             for p in workloads.decode5("cuda")]
    _run(specs, 1, "decode5")


def test_list_attn_q_b_fused_without_xq():
    d = workloads.attn_q_b("cuda")
    _run([dict(in_dim=1024, out_dim=32768, mode="x", w=d["w"], x=d["x"])], 1, "attn_q_b")


def test_list_router_and_shared_expert_gate_up():
    """One activation row feeding the router and the shared expert's gate and up."""
    specs = [dict(in_dim=4096, out_dim=256, mode="x+xq"),
             dict(in_dim=4096, out_dim=2048, mode="x", share=0),
             dict(in_dim=4096, out_dim=2048, mode="x+xq", share=0)]
    _run(specs, 1, "router_shared")


def test_list_mixed_paths():
    """Fused, pre-quantized, x_q-only, generic-fallback and off-list shapes in one call."""
    specs = [dict(in_dim=1024, out_dim=100, mode="x"),        # fused, 48 pairs
             dict(in_dim=2048, out_dim=77, mode="x+xq"),      # 96 pairs > LDS: own quantizer launch
             dict(in_dim=96, out_dim=19, mode="x+xq"),        # odd block count: generic kernel
             dict(in_dim=12288, out_dim=33, mode="xq"),       # 3 chunks per wave: own launch
             dict(in_dim=4096, out_dim=50, mode="xq"),        # list, reads x_q
             dict(in_dim=64, out_dim=65, mode="x"),           # fused, one pair per row
             dict(in_dim=8192, out_dim=40, mode="x+xq"),      # 2 waves per row
             dict(in_dim=16384, out_dim=20, mode="xq"),       # 4 waves per row
             dict(in_dim=32768, out_dim=10, mode="x+xq")]     # 4 waves x 2 chunks
    _run(specs, 3, "mixed")


@pytest.mark.parametrize("n_tok", [2, 4, 5, 11, 12, 17, 40, 80])
def test_list_token_counts(n_tok):
    # n_tok * 16 pairs <= 64 fuses; 5 and 11 tokens pre-quantize and share
    # the list launch; from 12 tokens the items leave the weight-streaming
    # path (the skinny matrix-core kernel up to 64, the tiled GEMM above),
    # each as its own launch.
    specs = [dict(in_dim=1024, out_dim=300, mode="x+xq"),
             dict(in_dim=256, out_dim=129, mode="x+xq"),
             dict(in_dim=4096, out_dim=64, mode="xq")]
    _run(specs, n_tok, f"ntok{n_tok}")


@pytest.mark.parametrize("in_dim,n_tok", [(64, 1), (128, 3), (256, 4), (512, 2), (1024, 1),
                                          (512, 3), (1024, 2), (2048, 1), (4096, 1)])
def test_list_one_item_fused(in_dim, n_tok):
    # One item with fp32 rows runs the dedicated fused kernel: with at most 16
    # pairs of x every wave quantizes the rows itself, above that the
    # workgroup shares one copy.  x_q is written too; 200 rows leave a ragged
    # last tile.
    _run([dict(in_dim=in_dim, out_dim=200, mode="x+xq")], n_tok, f"one{in_dim}x{n_tok}")


@pytest.mark.parametrize("out_dim", [1, 3, 17, 1000])
def test_list_ragged_rows_every_shape(out_dim):
    specs = [dict(in_dim=k, out_dim=out_dim, mode="x+xq" if k <= 4096 else "xq")
             for k in (64, 128, 256, 512, 1024, 2048, 4096, 8192, 16384, 24576, 32768)]
    _run(specs[:8], 1, f"ragged{out_dim}a")
    _run(specs[8:], 1, f"ragged{out_dim}b")


@pytest.mark.parametrize("out_dim,n_tok", [(513, 1), (1023, 2), (1024, 5)])
def test_list_wide_rows_two_row_groups(out_dim, n_tok):
    # 32768-wide rows take two row groups per workgroup from 511 rows on, their
    # four chunks per wave passing through the wave's two staging regions in
    # turn; an odd row count leaves the last workgroup's second row past the end.
    specs = [dict(in_dim=32768, out_dim=out_dim, mode="xq"),
             dict(in_dim=4096, out_dim=300, mode="x+xq")]
    _run(specs, n_tok, f"wide{out_dim}x{n_tok}")


def test_list_sixteen_items():
    dims = [64, 128, 256, 512, 1024, 2048, 4096, 4096, 1024, 512, 256, 128, 64, 2048, 1024, 8192]
    specs = [dict(in_dim=k, out_dim=37 + 5 * i, mode=("x", "x+xq", "xq")[i % 3] if k <= 4096 else "xq")
             for i, k in enumerate(dims)]
    assert len(specs) == _q8().LIST_MAX
    _run(specs, 1, "sixteen")


def test_list_special_values_fused():
    """Zero, non-finite and binary16-overflowing blocks through the in-launch quantizer."""
    x = workloads.normal((1, 1024), 1.0, "cpu", "list_special")
    x[0, 0:32] = 0.0
    x[0, 40] = float("nan")
    x[0, 70] = float("inf")
    x[0, 128:160] = 8321040.0
    x[0, 160:192] = 2.0 ** -149
    x[0, 200] = 127 * 2.0 ** -20
    x[0, 256:288:2] = -0.0
    d = np.float32(np.float32(3.3) / np.float32(127.0))
    x[0, 300] = 3.3
    x[0, 301] = float(np.float32(2.5 * np.float64(d)))    # tie in the quotient
    _run([dict(in_dim=1024, out_dim=200, mode="x+xq", x=x),
          dict(in_dim=1024, out_dim=64, mode="x", x=x)], 1, "special")


def _special_pattern(tag):
    """1024 values: a zero block, NaN, Inf, binary16-overflowing, subnormal
    and tiny-scale blocks, signed zeros and a tie in the quotient x/d."""
    x = workloads.normal((1, 1024), 1.0, "cpu", "list_special", tag)
    x[0, 0:32] = 0.0
    x[0, 40] = float("nan")
    x[0, 70] = float("inf")
    x[0, 128:160] = 8321040.0
    x[0, 160:192] = 2.0 ** -149
    x[0, 200] = 127 * 2.0 ** -20
    x[0, 256:288:2] = -0.0
    d = np.float32(np.float32(3.3) / np.float32(127.0))
    x[0, 300] = 3.3
    x[0, 301] = float(np.float32(2.5 * np.float64(d)))    # tie in the quotient
    x[0, 520] = -float("inf")
    x[0, 600:632] = -8321040.0
    x[0, 800] = -3.3
    x[0, 801] = -float(np.float32(2.5 * np.float64(d)))   # negative tie
    return x


@pytest.mark.parametrize("in_dim,n_tok", [(1024, 1), (512, 2), (256, 4)])
def test_list_special_values_one_item_wave(in_dim, n_tok):
    """The same special values through the one-item fused kernel whose waves
    each quantize the whole x (at most 16 pairs): the headline decode path."""
    x = _special_pattern("wave").reshape(n_tok, in_dim).contiguous()
    _run([dict(in_dim=in_dim, out_dim=200, mode="x+xq", x=x)], n_tok, f"special_wave{in_dim}")


def test_list_graph_replay_matches_eager():
    """The call is capturable: replays equal the eager result every time."""
    q8 = _q8()
    specs = workloads.decode5("cuda")
    items, outs = [], []
    for p in specs:
        wq = q8.q8_0_quantize_act(p["w"])
        out = torch.empty((1, p["out_dim"]), device="cuda")
        xq = torch.empty((1, q8.row_bytes(p["in_dim"])), dtype=torch.uint8, device="cuda")
        items.append(dict(out=out, w=wq, x=p["x"], x_q=xq, in_dim=p["in_dim"], out_dim=p["out_dim"]))
        outs.append(out)
    q8.q8_0_matmul_list(items, 1)
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            q8.q8_0_matmul_list(items, 1)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o.view(torch.int32), e.view(torch.int32)), f"replay {rep} differs"


def _random_calls(n_calls, seed):
    """Seeded list calls: 1-16 items of mixed in_dim (any multiple of 32 up to
    8192, and the 16384/32768 rows), ragged out_dim, every x mode the call
    accepts for the item; the oracle's work per call is bounded."""
    rng = np.random.default_rng(seed)
    calls = []
    while len(calls) < n_calls:
        n_tok = int(rng.choice([1, 1, 2, 4, 11, 12, 16, 40]))
        specs, work = [], 0
        for _ in range(int(rng.integers(1, 17))):
            r = rng.integers(0, 4)
            k = (32 * int(rng.integers(1, 257)) if r == 0 else
                 64 * 2 ** int(rng.integers(0, 8)) if r == 1 else
                 1024 * int(rng.integers(1, 9)) if r == 2 else int(rng.choice([16384, 32768])))
            n = int(rng.integers(1, 1500))
            # x without x_q only where the call quantizes inside its launch.
            fused = 64 <= k <= 4096 and k & (k - 1) == 0 and n_tok * k <= 4096
            modes = ["x", "x+xq", "xq"] if fused else ["x+xq", "xq"]
            specs.append(dict(in_dim=k, out_dim=n, mode=str(rng.choice(modes))))
            work += k * n * n_tok
        if work <= 2e8:
            calls.append((n_tok, specs))
    return calls


@pytest.mark.parametrize("case", range(12))
def test_list_random_calls(case):
    n_tok, specs = _random_calls(12, 77)[case]
    _run(specs, n_tok, f"random{case}")
