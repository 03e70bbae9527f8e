"""GPU parity for q8_0_matmul against the oracle, for every kernel variant.

Inputs are drawn by `workloads`, quantized on both sides independently (the
GPU quantizer for the GPU path, the oracle's for the oracle; the bytes are
also compared), then the fp32 outputs are checked to the stated tolerance and
the debug block sums bit-exactly.
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


def _prep(w, x):
    """Quantize on the GPU and, independently, with the oracle; compare bytes."""
    q8 = _q8()
    wq = q8.q8_0_quantize_act(w.cuda().contiguous())
    xq = q8.q8_0_quantize_act(x.cuda().contiguous())
    torch.cuda.synchronize()
    wq_o, xq_o = oracle_quantize(w), oracle_quantize(x)
    assert np.array_equal(cpu_u8(wq), wq_o), "weight quantization differs"
    assert np.array_equal(cpu_u8(xq), xq_o), "activation quantization differs"
    return wq, xq, wq_o, xq_o


def _run_and_check(wq, xq, wq_o, xq_o, in_dim, out_dim, n_tok, variant, split=0, where=""):
    q8 = _q8()
    say(f"[matmul] {where} in={in_dim} out={out_dim} n_tok={n_tok} variant={variant} split={split}")
    out = torch.full((n_tok, out_dim), float("nan"), device="cuda")   # poisoned
    ws = torch.empty(max(q8.q8_0_matmul_workspace_bytes(in_dim, out_dim, n_tok),
                         16 * out_dim * n_tok * 4 if split else 1), dtype=torch.uint8, device="cuda")
    got, bs = q8.q8_0_matmul_debug(wq, xq, in_dim, out_dim, n_tok, variant=variant, split_k=split,
                                   out=out, workspace=ws)
    torch.cuda.synchronize()
    ref, mag, rbs = oracle.matmul(wq_o, xq_o, in_dim, want_blocksums=True)
    assert_close(got.cpu().numpy(), ref, mag, where)
    assert np.array_equal(bs.cpu().numpy(), rbs), f"{where}: block sums differ"
    return got


VARIANTS = [1, 2, 3]


@pytest.mark.parametrize("variant", VARIANTS)
def test_tiny_workload_all_variants(variant):
    d = workloads.tiny("cuda")
    wq, xq, wq_o, xq_o = _prep(d["w"], d["x"])
    _run_and_check(wq, xq, wq_o, xq_o, 256, 128, 4, variant, where="tiny")


@pytest.mark.parametrize("in_dim", [64, 128, 256, 512, 1024, 2048, 4096, 8192, 12288, 16384,
                                    32768, 49152, 65536])
def test_matvec_shapes(in_dim):
    out_dim, n_tok = 37, 3
    w = workloads.normal((out_dim, in_dim), 0.02, "cuda", "mv", in_dim, "w")
    x = workloads.normal((n_tok, in_dim), 1.0, "cuda", "mv", in_dim, "x")
    wq, xq, wq_o, xq_o = _prep(w, x)
    _run_and_check(wq, xq, wq_o, xq_o, in_dim, out_dim, n_tok, 2, where="matvec")
    _run_and_check(wq, xq, wq_o, xq_o, in_dim, out_dim, n_tok, 1, where="generic")


@pytest.mark.parametrize("in_dim", [32, 96, 160, 3072, 4160])
def test_generic_only_shapes(in_dim):
    q8 = _q8()
    out_dim, n_tok = 19, 2
    w = workloads.normal((out_dim, in_dim), 0.02, "cuda", "gen", in_dim, "w")
    x = workloads.normal((n_tok, in_dim), 1.0, "cuda", "gen", in_dim, "x")
    wq, xq, wq_o, xq_o = _prep(w, x)
    assert q8.q8_0_matmul_plan(in_dim, out_dim, n_tok, 0)[0] in (1, 2)
    _run_and_check(wq, xq, wq_o, xq_o, in_dim, out_dim, n_tok, 0, where="auto")


@pytest.mark.parametrize("out_dim,n_tok,in_dim,split", [
    (300, 150, 1152, 1), (300, 150, 1152, 3), (128, 64, 4096, 1), (77, 16, 2048, 4),
    (256, 257, 512, 2), (33, 1, 1024, 1), (130, 70, 8192, 16)])
def test_mfma_ragged(out_dim, n_tok, in_dim, split):
    w = workloads.normal((out_dim, in_dim), 0.02, "cuda", "mf", out_dim, in_dim, "w")
    x = workloads.normal((n_tok, in_dim), 1.0, "cuda", "mf", n_tok, in_dim, "x")
    wq, xq, wq_o, xq_o = _prep(w, x)
    _run_and_check(wq, xq, wq_o, xq_o, in_dim, out_dim, n_tok, 3, split, where="mfma")


def test_subnormal_and_nan_scales():
    # Tiny weights give binary16-subnormal scales; a NaN-marked x block must
    # poison exactly the outputs of its token on every path.
    in_dim, out_dim, n_tok = 512, 64, 20
    w = workloads.normal((out_dim, in_dim), 2e-7, "cuda", "sub", "w")
    x = workloads.normal((n_tok, in_dim), 1.0, "cuda", "sub", "x")
    x[3, 17] = float("nan")
    wq, xq, wq_o, xq_o = _prep(w, x)
    for v in VARIANTS:
        _run_and_check(wq, xq, wq_o, xq_o, in_dim, out_dim, n_tok, v, where=f"subnormal v{v}")


def test_attn_q_b_full():
    q8 = _q8()
    d = workloads.attn_q_b("cuda")
    wq, xq, wq_o, xq_o = _prep(d["w"], d["x"])
    assert q8.q8_0_matmul_plan(1024, 32768, 1, 0) == (2, 1)
    say("[matmul] attn_q_b auto")
    got = q8.q8_0_matmul(wq, xq, 1024, 32768, 1)
    torch.cuda.synchronize()
    ref, mag, _ = oracle.matmul(wq_o, xq_o, 1024)
    assert_close(got.cpu().numpy(), ref, mag, "attn_q_b")
    for v in VARIANTS:
        _run_and_check(wq, xq, wq_o, xq_o, 1024, 32768, 1, v, where=f"attn_q_b v{v}")


def test_decode5_full():
    q8 = _q8()
    for p in workloads.decode5("cuda"):
        wq, xq, wq_o, xq_o = _prep(p["w"], p["x"])
        say(f"[matmul] decode5 {p['name']}")
        got = q8.q8_0_matmul(wq, xq, p["in_dim"], p["out_dim"], 1)
        torch.cuda.synchronize()
        ref, mag, _ = oracle.matmul(wq_o, xq_o, p["in_dim"])
        assert_close(got.cpu().numpy(), ref, mag, p["name"])


@pytest.mark.parametrize("name", ["prefill_a", "prefill_b"])
def test_prefill_full_sampled(name):
    """Full-size launch as timed by the benchmark; the oracle checks a sample of
    64 tokens x 96 output rows, plus every quantized activation byte."""
    q8 = _q8()
    d = workloads.prefill(name, "cuda")
    k, n, t = d["in_dim"], d["out_dim"], d["n_tok"]
    wq = q8.q8_0_quantize_act(d["w"])
    xq = q8.q8_0_quantize_act(d["x"])
    say(f"[matmul] {name} full plan={q8.q8_0_matmul_plan(k, n, t, 1 << 40)}")
    got = q8.q8_0_matmul(wq, xq, k, n, t)
    torch.cuda.synchronize()
    assert q8.q8_0_matmul_plan(k, n, t, 1 << 40)[0] == 3
    rng = np.random.default_rng(5)
    toks = np.sort(rng.choice(t, 64, replace=False))
    rows = np.sort(rng.choice(n, 96, replace=False))
    xq_o = oracle_quantize(d["x"][torch.as_tensor(toks, device="cuda")])
    wq_o = oracle_quantize(d["w"][torch.as_tensor(rows, device="cuda")])
    assert np.array_equal(cpu_u8(xq)[toks], xq_o)
    assert np.array_equal(cpu_u8(wq)[rows], wq_o)
    ref, mag, _ = oracle.matmul(wq_o, xq_o, k)
    assert_close(got.cpu().numpy()[np.ix_(toks, rows)], ref, mag, name)


def test_prefill_slices_blocksums():
    # Debug-mode block sums on a slice of each prefill workload (first 160
    # tokens x 192 rows, whole K), through the MFMA kernel with split-K.
    for name in ("prefill_a", "prefill_b"):
        d = workloads.prefill(name, "cuda", rows=192, tokens=160)
        wq, xq, wq_o, xq_o = _prep(d["w"], d["x"])
        _run_and_check(wq, xq, wq_o, xq_o, d["in_dim"], 192, 160, 3, 2, where=f"{name} slice")


def test_deterministic_and_sign_flip():
    q8 = _q8()
    in_dim, out_dim = 2048, 512
    for n_tok in (1, 5, 80):
        w = workloads.normal((out_dim, in_dim), 0.02, "cuda", "det", "w")
        x = workloads.normal((n_tok, in_dim), 1.0, "cuda", "det", n_tok)
        wq = q8.q8_0_quantize_act(w)
        xq = q8.q8_0_quantize_act(x)
        xqn = q8.q8_0_quantize_act(-x)
        a = q8.q8_0_matmul(wq, xq, in_dim, out_dim, n_tok)
        b = q8.q8_0_matmul(wq, xq, in_dim, out_dim, n_tok)
        c = q8.q8_0_matmul(wq, xqn, in_dim, out_dim, n_tok)
        torch.cuda.synchronize()
        assert torch.equal(a, b)
        assert torch.equal(c, -a)


def test_empty_and_errors():
    q8 = _q8()
    wq = torch.zeros((4, 34), dtype=torch.uint8, device="cuda")
    xq = torch.zeros((1, 34), dtype=torch.uint8, device="cuda")
    out = torch.empty((0, 4), device="cuda")
    q8.q8_0_matmul(wq, xq, 32, 4, 0, out=out)          # n_tok == 0: no-op
    with pytest.raises(q8.Q8Error) as e:
        q8.q8_0_matmul(wq, xq, 33, 4, 1)
    assert e.value.code == q8.Q8_0_EINVAL
    with pytest.raises(q8.Q8Error) as e:
        q8.q8_0_matmul_debug(wq, xq, 32, 4, 1, variant=2)  # matvec needs whole pairs
    assert e.value.code == q8.Q8_0_EINVAL
