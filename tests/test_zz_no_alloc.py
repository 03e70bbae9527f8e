"""GPU check of q8_0_moe_grouped_noalloc, the grouped expert matmul whose
routing tables live in the library's static device array instead of caller
workspace.  It is called through the C ABI (ctypes) and compared with
q8_0_moe_grouped on the same inputs -- bit for bit, since both run the same
kernels -- and with the oracle, within the stated tolerance.  Two calls in a
row, the second with a smaller routing shape, show that the shared array's
contents from the first call do not leak into the second.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.helpers import assert_close, cpu_u8, oracle_quantize, say

pytestmark = pytest.mark.gpu


def _case(q8, in_dim, out_dim, n_expert, n_tok, n_used, seed, x_rows):
    ws_f = [workloads.normal((out_dim, in_dim), 0.02, "cuda", "noalloc", seed, e)
            for e in range(n_expert)]
    wq = [q8.q8_0_quantize_act(w) for w in ws_f]
    g = torch.Generator().manual_seed(seed)
    sel = torch.stack([torch.randperm(n_expert, generator=g)[:n_used] for _ in range(n_tok)])
    sel = sel.to(torch.int32)
    rows = n_tok * n_used if x_rows else n_tok
    x = workloads.normal((rows, in_dim), 1.0, "cuda", "noalloc", seed, "x")
    xq = q8.q8_0_quantize_act(x)
    torch.cuda.synchronize()
    wq_o = [oracle_quantize(w) for w in ws_f]
    xq_o = oracle_quantize(x)
    for a, b in zip(wq, wq_o):
        assert np.array_equal(cpu_u8(a), b)
    assert np.array_equal(cpu_u8(xq), xq_o)
    return wq, sel, xq, wq_o, xq_o


def _noalloc_raw(q8, table, n_expert, sel, xq, in_dim, out_dim, x_rows, out, inv):
    """The C entry point, called directly through ctypes."""
    n_tok, n_used = sel.shape
    lib = q8.raw_library()
    return lib.q8_0_moe_grouped_noalloc(
        ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(table.data_ptr()), n_expert, in_dim,
        out_dim, ctypes.c_void_p(sel.data_ptr()), n_used, ctypes.c_void_p(xq.data_ptr()),
        x_rows, n_tok, ctypes.c_void_p(inv.data_ptr()),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def test_noalloc_matches_workspace_call_twice_then_smaller():
    import q8_quantized_matmul_amd as q8
    # First call: 256 experts, 64 tokens x 8 slots (the moe workload's routing
    # shape) at a reduced matrix size; second: fewer experts, tokens and slots.
    shapes = [(1024, 192, 256, 64, 8, 0, 501), (512, 96, 12, 9, 3, 1, 502)]
    for in_dim, out_dim, n_expert, n_tok, n_used, x_rows, seed in shapes:
        say(f"[noalloc] in={in_dim} out={out_dim} E={n_expert} T={n_tok} k={n_used} "
            f"x_rows={x_rows}")
        wq, sel, xq, wq_o, xq_o = _case(q8, in_dim, out_dim, n_expert, n_tok, n_used, seed, x_rows)
        table = q8.expert_table(wq)
        sel_d = sel.cuda()
        out = torch.full((n_tok, n_used, out_dim), float("nan"), device="cuda")
        inv = torch.full((1,), -7, dtype=torch.int32, device="cuda")
        rc = _noalloc_raw(q8, table, n_expert, sel_d, xq, in_dim, out_dim, x_rows, out, inv)
        assert rc == 0, q8.q8_0_strerror(rc)
        ref_gpu, ws = q8.q8_0_moe_grouped(table, n_expert, sel_d, xq, in_dim, out_dim, x_rows)
        torch.cuda.synchronize()
        assert int(inv.item()) == 0
        assert q8.moe_invalid_count(ws) == 0
        assert torch.equal(out, ref_gpu), "static-scratch call differs from the workspace call"
        ref, mag, bad = oracle.moe_grouped(wq_o, sel.numpy(), xq_o, in_dim, out_dim, x_rows)
        assert bad == 0
        assert_close(out.cpu().numpy(), ref, mag, "noalloc vs oracle")


def test_noalloc_invalid_ids_counted():
    import q8_quantized_matmul_amd as q8
    in_dim, out_dim, n_expert, n_tok, n_used = 256, 40, 6, 5, 2
    wq, sel, xq, wq_o, xq_o = _case(q8, in_dim, out_dim, n_expert, n_tok, n_used, 503, 0)
    sel = sel.clone()
    sel[0, 1] = 9
    sel[3, 0] = -1
    table = q8.expert_table(wq)
    inv = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = q8.q8_0_moe_grouped_noalloc(table, n_expert, sel.cuda(), xq, in_dim, out_dim, 0,
                                      n_invalid=inv)
    torch.cuda.synchronize()
    assert int(inv.item()) == 2
    ref, mag, bad = oracle.moe_grouped(wq_o, sel.numpy(), xq_o, in_dim, out_dim, 0)
    assert bad == 2
    assert_close(out.cpu().numpy(), ref, mag, "noalloc invalid ids")
