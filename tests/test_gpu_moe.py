"""GPU parity for q8_0_moe_grouped (routing on the GPU + grouped expert matmul)."""
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


def _small_case(in_dim, out_dim, n_expert, n_tok, n_used, seed, x_rows):
    q8 = _q8()
    ws_f = [workloads.normal((out_dim, in_dim), 0.02, "cuda", "moe_t", seed, e) for e in range(n_expert)]
    wq = [q8.q8_0_quantize_act(w) for w in ws_f]
    g = torch.Generator().manual_seed(seed)
    sel = torch.stack([torch.randperm(n_expert, generator=g)[:n_used] for _ in range(n_tok)])
    sel = sel.to(torch.int32)
    rows = n_tok * n_used if x_rows else n_tok
    x = workloads.normal((rows, in_dim), 1.0, "cuda", "moe_t", seed, "x")
    xq = q8.q8_0_quantize_act(x)
    torch.cuda.synchronize()
    wq_o = [oracle_quantize(w) for w in ws_f]
    xq_o = oracle_quantize(x)
    for a, b in zip(wq, wq_o):
        assert np.array_equal(cpu_u8(a), b)
    assert np.array_equal(cpu_u8(xq), xq_o)
    return wq, sel, xq, wq_o, xq_o


@pytest.mark.parametrize("in_dim,out_dim,n_expert,n_tok,n_used,x_rows", [
    (256, 96, 8, 5, 3, 0), (256, 96, 8, 5, 3, 1), (2048, 130, 16, 9, 4, 1),
    (4096, 64, 32, 40, 8, 0), (96, 40, 5, 6, 2, 0), (1024, 70, 3, 33, 3, 1)])
def test_moe_small(in_dim, out_dim, n_expert, n_tok, n_used, x_rows):
    q8 = _q8()
    wq, sel, xq, wq_o, xq_o = _small_case(in_dim, out_dim, n_expert, n_tok, n_used, in_dim + n_tok,
                                          x_rows)
    table = q8.expert_table(wq)
    say(f"[moe] in={in_dim} out={out_dim} E={n_expert} T={n_tok} k={n_used} x_rows={x_rows}")
    out = torch.full((n_tok, n_used, out_dim), float("nan"), device="cuda")
    got, bs, ws = q8.q8_0_moe_grouped_debug(table, n_expert, sel.cuda(), xq, in_dim, out_dim,
                                            x_rows, out=out)
    torch.cuda.synchronize()
    assert q8.moe_invalid_count(ws) == 0
    ref, mag, bad = oracle.moe_grouped(wq_o, sel.numpy(), xq_o, in_dim, out_dim, x_rows)
    assert bad == 0
    assert_close(got.cpu().numpy(), ref, mag, "moe small")
    # Block sums of each pair against the oracle's dense matmul of that pair.
    bsn = bs.cpu().numpy().reshape(n_tok, n_used, out_dim, -1)
    for t in range(n_tok):
        for j in range(n_used):
            row = t * n_used + j if x_rows else t
            _, _, rbs = oracle.matmul(wq_o[int(sel[t, j])], xq_o[row:row + 1], in_dim,
                                      want_blocksums=True)
            assert np.array_equal(bsn[t, j], rbs[0])
    # Deterministic.
    got2, _ = q8.q8_0_moe_grouped(table, n_expert, sel.cuda(), xq, in_dim, out_dim, x_rows)
    torch.cuda.synchronize()
    assert torch.equal(got, got2)


@pytest.mark.parametrize("in_dim,out_dim,n_expert,x_rows", [(4096, 1029, 16, 0), (2048, 2051, 16, 1)])
def test_moe_four_row_groups_ragged(in_dim, out_dim, n_expert, x_rows):
    # Enough tiles for four row groups per wave slot, whose four row sums per
    # lane are reduced together (64-lane rows at in_dim 4096, 32-lane rows at
    # 2048); the row counts leave a ragged last tile.
    q8 = _q8()
    n_tok, n_used = 8, 4
    wq, sel, xq, wq_o, xq_o = _small_case(in_dim, out_dim, n_expert, n_tok, n_used, in_dim + out_dim,
                                          x_rows)
    table = q8.expert_table(wq)
    say(f"[moe] four row groups in={in_dim} out={out_dim} E={n_expert} x_rows={x_rows}")
    out = torch.full((n_tok, n_used, out_dim), float("nan"), device="cuda")
    got, _ = q8.q8_0_moe_grouped(table, n_expert, sel.cuda(), xq, in_dim, out_dim, x_rows, out=out)
    torch.cuda.synchronize()
    ref, mag, bad = oracle.moe_grouped(wq_o, sel.numpy(), xq_o, in_dim, out_dim, x_rows)
    assert bad == 0
    assert_close(got.cpu().numpy(), ref, mag, "moe four row groups")
    got2, _ = q8.q8_0_moe_grouped(table, n_expert, sel.cuda(), xq, in_dim, out_dim, x_rows)
    torch.cuda.synchronize()
    assert torch.equal(got, got2)


def test_moe_invalid_ids_and_duplicates():
    q8 = _q8()
    in_dim, out_dim, n_expert, n_tok, n_used = 512, 48, 6, 7, 3
    wq, sel, xq, wq_o, xq_o = _small_case(in_dim, out_dim, n_expert, n_tok, n_used, 99, 0)
    sel = sel.clone()
    sel[1, 2] = 6          # out of range
    sel[4, 0] = -3         # out of range
    sel[5, 1] = sel[5, 0]  # duplicate id in one token's list
    table = q8.expert_table(wq)
    got, ws = q8.q8_0_moe_grouped(table, n_expert, sel.cuda(), xq, in_dim, out_dim, 0)
    torch.cuda.synchronize()
    assert q8.moe_invalid_count(ws) == 2
    ref, mag, bad = oracle.moe_grouped(wq_o, sel.numpy(), xq_o, in_dim, out_dim, 0)
    assert bad == 2
    assert_close(got.cpu().numpy(), ref, mag, "moe invalid")


def _moe_stack(q8, which, E, rows, cols):
    st = torch.empty((E, rows, q8.row_bytes(cols)), dtype=torch.uint8, device="cuda")
    for e in range(E):
        q8.q8_0_quantize_act(workloads.moe_expert(e, which, "cuda"), out=st[e])
    return st


@pytest.mark.parametrize("which", ["gate", "up", "down"])
def test_moe_workload_full(which):
    """The benchmark's MoE workload at full size (256 experts, 64 tokens x 8
    slots), one projection per test: every (token, slot) pair's whole output
    row against the oracle, and every touched expert's quantized bytes."""
    q8 = _q8()
    cfg = workloads.MOE
    E, k, T, D, F = cfg["n_expert"], cfg["n_used"], cfg["n_tok"], cfg["d_model"], cfg["d_ff"]
    in_dim, out_dim = (D, F) if which != "down" else (F, D)
    x_rows = 1 if which == "down" else 0
    sel = workloads.moe_routing()
    x, mid = workloads.moe_acts("cuda")
    src_f = mid[: T * k] if x_rows else x
    src = q8.q8_0_quantize_act(src_f)
    say(f"[moe] full {which}: quantizing 256 experts")
    st = _moe_stack(q8, which, E, out_dim, in_dim)
    got, ws = q8.q8_0_moe_grouped(q8.expert_table(st), E, sel.cuda(), src, in_dim, out_dim, x_rows)
    torch.cuda.synchronize()
    assert q8.moe_invalid_count(ws) == 0
    touched = sorted(set(sel.reshape(-1).tolist()))
    dummy = np.zeros((1, q8.row_bytes(in_dim)), dtype=np.uint8)
    mats = [dummy] * E
    with oracle.threads():
        src_o = oracle_quantize(src_f)
        assert np.array_equal(cpu_u8(src), src_o)
        for e in touched:
            w_o = oracle_quantize(workloads.moe_expert(e, which, "cuda"))
            assert np.array_equal(cpu_u8(st[e]), w_o), f"expert {e} bytes"
            mats[e] = w_o
        say(f"[moe] full {which}: oracle over {T * k} pairs, {len(touched)} experts")
        ref, mag, bad = oracle.moe_grouped(mats, sel.numpy(), src_o, in_dim, out_dim, x_rows)
    assert bad == 0
    assert_close(got.cpu().numpy(), ref, mag, f"moe {which} full")


@pytest.mark.parametrize("which", ["gate", "up", "down"])
def test_moe_shared_expert_full(which):
    """The shared expert of the MoE workload: a dense q8_0_matmul at 64 tokens
    (the skinny matrix-core kernel, split-K through its workspace), every
    output against the oracle."""
    q8 = _q8()
    cfg = workloads.MOE
    k, T, D, F = cfg["n_used"], cfg["n_tok"], cfg["d_model"], cfg["d_ff"]
    in_dim, out_dim = (D, F) if which != "down" else (F, D)
    x, mid = workloads.moe_acts("cuda")
    src_f = mid[T * k:] if which == "down" else x
    w = workloads.moe_expert(-1, which, "cuda")
    wq = q8.q8_0_quantize_act(w)
    xq = q8.q8_0_quantize_act(src_f)
    ws = q8.matmul_workspace(in_dim, out_dim, T)
    plan = q8.q8_0_matmul_plan(in_dim, out_dim, T, ws.numel())
    say(f"[moe] shared {which} plan={plan}")
    out = torch.full((T, out_dim), float("nan"), device="cuda")
    got = q8.q8_0_matmul(wq, xq, in_dim, out_dim, T, out=out, workspace=ws)
    torch.cuda.synchronize()
    with oracle.threads():
        wq_o = oracle_quantize(w)
        xq_o = oracle_quantize(src_f)
        assert np.array_equal(cpu_u8(wq), wq_o) and np.array_equal(cpu_u8(xq), xq_o)
        ref, mag, _ = oracle.matmul(wq_o, xq_o, in_dim)
    assert_close(got.cpu().numpy(), ref, mag, f"shared {which}")


@pytest.mark.parametrize("n_expert,n_tok,n_used,n_bad", [
    (256, 64, 8, 0), (5000, 300, 8, 7), (3, 700, 3, 2), (8192, 2, 1, 0), (1, 5, 2, 1)])
def test_moe_routing_tables(n_expert, n_tok, n_used, n_bad):
    # The routing tables are index work: compared exactly with their plain
    # definitions (counts = histogram of the valid ids, offsets = its exclusive
    # prefix sum, pairs = the pair ids in a stable sort by expert id).  The
    # int32 layout of the workspace: [0] invalid-id count, counts at 16,
    # offsets (n_expert + 1) after them, then the pair list.  Several
    # 1024-pair chunks, experts per lane above one, duplicates and invalid ids.
    q8 = _q8()
    rng = np.random.default_rng(n_expert * 31 + n_tok)
    sel = rng.integers(0, n_expert, size=(n_tok, n_used)).astype(np.int32)
    flat = sel.reshape(-1)
    bad_at = rng.choice(flat.size, n_bad, replace=False)
    flat[bad_at] = np.where(np.arange(n_bad) % 2 == 0, n_expert + 3, -1)
    out_dim, in_dim = 4, 32
    stack = torch.zeros((n_expert, out_dim, q8.row_bytes(in_dim)), dtype=torch.uint8, device="cuda")
    xq = torch.zeros((n_tok, q8.row_bytes(in_dim)), dtype=torch.uint8, device="cuda")
    say(f"[moe routing] E={n_expert} T={n_tok} k={n_used} bad={n_bad}")
    _, ws = q8.q8_0_moe_grouped(q8.expert_table(stack), n_expert, torch.from_numpy(sel).cuda(),
                                xq, in_dim, out_dim, 0)
    torch.cuda.synchronize()
    got = ws.cpu().view(torch.int32).numpy()
    valid = (flat >= 0) & (flat < n_expert)
    counts = np.bincount(flat[valid], minlength=n_expert)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    pairs = np.argsort(np.where(valid, flat, n_expert), kind="stable")[:int(valid.sum())]
    c0, o0 = 16, 16 + n_expert
    p0 = o0 + n_expert + 1
    assert got[0] == n_bad
    assert np.array_equal(got[c0:c0 + n_expert], counts)
    assert np.array_equal(got[o0:o0 + n_expert + 1], offsets)
    assert np.array_equal(got[p0:p0 + pairs.size], pairs)


def _random_moe(n_cases, seed):
    """Seeded grouped calls: any in_dim multiple of 32 up to 4096 (both the
    weight-streaming and the generic grouped kernels), 1-40 experts, 1-150
    tokens, either x layout; the oracle's work per case is bounded."""
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n_cases:
        in_dim = (32 * int(rng.integers(1, 129)) if rng.integers(0, 2) else
                  64 * 2 ** int(rng.integers(0, 7)))
        out_dim = int(rng.integers(1, 300))
        n_expert = int(rng.integers(1, 41))
        n_used = int(rng.integers(1, min(8, n_expert) + 1))
        n_tok = int(rng.choice([1, 2, 7, 16, 17, 40, 150]))
        if in_dim * out_dim * n_tok * n_used <= 6e7:
            cases.append((in_dim, out_dim, n_expert, n_tok, n_used, int(rng.integers(0, 2))))
    return cases


@pytest.mark.parametrize("in_dim,out_dim,n_expert,n_tok,n_used,x_rows", _random_moe(12, 31))
def test_moe_random_shapes(in_dim, out_dim, n_expert, n_tok, n_used, x_rows):
    q8 = _q8()
    wq, sel, xq, wq_o, xq_o = _small_case(in_dim, out_dim, n_expert, n_tok, n_used,
                                          in_dim * 7 + n_tok, x_rows)
    say(f"[moe random] in={in_dim} out={out_dim} E={n_expert} T={n_tok} k={n_used} x_rows={x_rows}")
    out = torch.full((n_tok, n_used, out_dim), float("nan"), device="cuda")
    got, ws = q8.q8_0_moe_grouped(q8.expert_table(wq), n_expert, sel.cuda(), xq, in_dim, out_dim,
                                  x_rows, out=out)
    torch.cuda.synchronize()
    assert q8.moe_invalid_count(ws) == 0
    ref, mag, bad = oracle.moe_grouped(wq_o, sel.numpy(), xq_o, in_dim, out_dim, x_rows)
    assert bad == 0
    assert_close(got.cpu().numpy(), ref, mag, "moe random")
