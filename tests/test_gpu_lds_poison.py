"""LDS poisoning: no kernel of the path may read LDS it has not written.

A kernel that reads LDS before writing it, or before the barrier that
publishes another wave's writes, computes from whatever the LDS held: the
leftovers of earlier launches, which usually make the bug invisible.  Here
the whole LDS of every compute unit is filled with a chosen 32-bit pattern
(q8_0_debug_poison_lds) right before the call under test, and each call runs
after several patterns (NaN bits, 0x7f bytes, zeros, ...); every output must
be bit-identical to the first run.  The first test checks the mechanism
itself: LDS left by the poisoning launch is what a later launch's workgroups
find.  Calls of several launches (the routed FFN) see the pattern in their
first launch; the later ones start from the LDS the earlier ones left.
"""
import pytest
import torch

import workloads
from tests.helpers import say

pytestmark = pytest.mark.gpu

PATTERNS = [0x00000000, 0xFFFFFFFF, 0x7F7F7F7F, 0x80000001, 0x3C00BC00]


def _q8():
    import q8_quantized_matmul_amd as q8
    return q8


def _mat(q8, rows, cols, *tag):
    return q8.q8_0_quantize_act(workloads.normal((rows, cols), 0.02, "cuda", "poison", *tag))


def _x(rows, cols, *tag):
    return workloads.normal((rows, cols), 1.0, "cuda", "poison_x", *tag)


@pytest.mark.parametrize("pattern", [0xFFFFFFFF, 0x12345678])
def test_poison_reaches_later_launches(pattern):
    q8 = _q8()
    wgs = 256
    seen = torch.zeros(wgs * q8.DEBUG_LDS_DWORDS, dtype=torch.int32, device="cuda")
    q8.q8_0_debug_poison_lds(pattern)
    q8.q8_0_debug_read_lds(seen, wgs)
    torch.cuda.synchronize()
    want = pattern - (1 << 32) if pattern >= (1 << 31) else pattern
    frac = (seen == want).double().mean().item()
    say(f"[poison] pattern {pattern:#010x}: {frac:.6f} of the read-back LDS holds it")
    assert frac == 1.0


def _matmul_case(in_dim, out_dim, n_tok, variant=None, blocksums=False):
    def make():
        q8 = _q8()
        w = _mat(q8, out_dim, in_dim, "w", in_dim, out_dim)
        xq = q8.q8_0_quantize_act(_x(n_tok, in_dim, "x", in_dim, n_tok))
        out = torch.empty((n_tok, out_dim), dtype=torch.float32, device="cuda")
        if variant is None:
            nb = q8.q8_0_matmul_workspace_bytes(in_dim, out_dim, n_tok)
            ws = q8.matmul_workspace(in_dim, out_dim, n_tok) if nb > 0 else None

            def call():
                q8.q8_0_matmul(w, xq, in_dim, out_dim, n_tok, out=out, workspace=ws)
                return [out]
        else:
            ws = q8.matmul_workspace(in_dim, out_dim, n_tok, variant=variant)

            def call():
                _, bs = q8.q8_0_matmul_debug(w, xq, in_dim, out_dim, n_tok, variant=variant,
                                             blocksums=blocksums, out=out, workspace=ws)
                return [out] + ([bs] if blocksums else [])
        return [out], call
    return make


def _quantize_case(n_tok, in_dim):
    def make():
        q8 = _q8()
        x = _x(n_tok, in_dim, "q", n_tok, in_dim)
        xq = torch.empty((n_tok, q8.row_bytes(in_dim)), dtype=torch.uint8, device="cuda")

        def call():
            q8.q8_0_quantize_act(x, out=xq)
            return [xq]
        return [xq], call
    return make


def _list_case(specs, n_tok):
    """specs: (in_dim, out_dim, fused) per item; fused items quantize x in the launch."""
    def make():
        q8 = _q8()
        items, outs = [], []
        for j, (k, n, fused) in enumerate(specs):
            w = _mat(q8, n, k, "l", j, k, n)
            x = _x(n_tok, k, "lx", j, k, n_tok)
            out = torch.empty((n_tok, n), dtype=torch.float32, device="cuda")
            xq = torch.empty((n_tok, q8.row_bytes(k)), dtype=torch.uint8, device="cuda")
            if fused:
                items.append(dict(out=out, w=w, x=x, x_q=xq, in_dim=k, out_dim=n))
                outs += [out, xq]
            else:
                q8.q8_0_quantize_act(x, out=xq)
                items.append(dict(out=out, w=w, x_q=xq, in_dim=k, out_dim=n))
                outs.append(out)

        def call():
            q8.q8_0_matmul_list(items, n_tok)
            return outs
        return [o for o in outs if o.dtype == torch.float32], call
    return make


def _moe_case(in_dim, out_dim, n_expert, n_tok, n_used, x_rows):
    def make():
        q8 = _q8()
        table_src = [_mat(q8, out_dim, in_dim, "e", e) for e in range(n_expert)]
        table = q8.expert_table(table_src)
        g = torch.Generator().manual_seed(n_expert * 131 + n_tok)
        sel = torch.stack([torch.randperm(n_expert, generator=g)[:n_used] for _ in range(n_tok)])
        sel = sel.to(torch.int32).cuda()
        rows = n_tok * n_used if x_rows else n_tok
        xq = q8.q8_0_quantize_act(_x(rows, in_dim, "mx", in_dim))
        out = torch.empty((n_tok, n_used, out_dim), dtype=torch.float32, device="cuda")
        ws = torch.zeros(q8.q8_0_moe_workspace_bytes(n_tok, n_used, n_expert), dtype=torch.uint8,
                         device="cuda")

        def call(keep=table_src):  # keep: the expert table points into these tensors
            q8.q8_0_moe_grouped(table, n_expert, sel, xq, in_dim, out_dim, x_rows, out=out,
                                workspace=ws)
            return [out, ws]
        return [out], call
    return make


def _ffn_case(d_model, d_ff, n_expert, n_tok, n_used):
    def make():
        q8 = _q8()
        tabs, keep = [], []
        for which, (rows, cols) in (("gate", (d_ff, d_model)), ("up", (d_ff, d_model)),
                                    ("down", (d_model, d_ff))):
            mats = [_mat(q8, rows, cols, which, e) for e in range(n_expert)]
            keep.append(mats)
            tabs.append(q8.expert_table(mats))
        g = torch.Generator().manual_seed(7 * n_expert + n_tok)
        sel = torch.stack([torch.randperm(n_expert, generator=g)[:n_used] for _ in range(n_tok)])
        sel = sel.to(torch.int32).cuda()
        wts = torch.rand((n_tok, n_used), generator=g).cuda()
        xq = q8.q8_0_quantize_act(_x(n_tok, d_model, "fx", d_model))
        pairs = n_tok * n_used
        out = torch.empty((n_tok, d_model), dtype=torch.float32, device="cuda")
        mid = torch.empty((pairs, d_ff), dtype=torch.float32, device="cuda")
        mid_q = torch.empty((pairs, q8.row_bytes(d_ff)), dtype=torch.uint8, device="cuda")
        y = torch.empty((pairs, d_model), dtype=torch.float32, device="cuda")
        ws = torch.zeros(max(q8.q8_0_moe_ffn_workspace_bytes(n_tok, n_used, n_expert, d_model,
                                                              d_ff), 256),
                         dtype=torch.uint8, device="cuda")

        def call(keep=keep):  # keep: the expert tables point into these tensors
            q8.q8_0_moe_ffn(tabs[0], tabs[1], tabs[2], n_expert, sel, wts, xq, d_model, d_ff,
                            10.0, out=out, mid=mid, mid_q=mid_q, y=y, workspace=ws)
            return [out, mid, mid_q, y]
        return [out, mid, y], call
    return make


def _cases():
    return {
        "quantize 64x4096": _quantize_case(64, 4096),
        "quantize 3x1056": _quantize_case(3, 1056),
        "matvec 1024->2048": _matmul_case(1024, 2048, 1),
        "matvec 4096->1000": _matmul_case(4096, 1000, 1),
        "matvec 32768->260": _matmul_case(32768, 260, 1),
        "matvec staged x 4096->1024, 5 tokens": _matmul_case(4096, 1024, 5),
        "skinny 4096->2048, 32 tokens": _matmul_case(4096, 2048, 32),
        "skinny 1024->520, 20 tokens, block sums": _matmul_case(1024, 520, 20, variant=4,
                                                                blocksums=True),
        "gemm four-tile 4096->512, 256 tokens": _matmul_case(4096, 512, 256),
        "gemm four-tile 2048->256, 256 tokens, block sums": _matmul_case(2048, 256, 256, variant=3,
                                                                         blocksums=True),
        "gemm ragged 1024->300, 130 tokens": _matmul_case(1024, 300, 130),
        "generic 96->70, 3 tokens, block sums": _matmul_case(96, 70, 3, variant=1,
                                                             blocksums=True),
        "list fused one item 1024->4096": _list_case([(1024, 4096, True)], 1),
        "list decode mix": _list_case([(4096, 1024, True), (4096, 512, False),
                                       (32768, 256, False), (1024, 4096, True),
                                       (4096, 256, True)], 1),
        "list 3 tokens": _list_case([(4096, 520, True), (2048, 300, False)], 3),
        "moe grouped": _moe_case(1024, 512, 16, 8, 4, 0),
        "moe grouped, x per pair": _moe_case(2048, 130, 8, 9, 3, 1),
        "moe routed ffn": _ffn_case(512, 256, 8, 6, 2),
    }


CASES = list(_cases().keys())


@pytest.mark.parametrize("case", CASES)
def test_outputs_do_not_depend_on_lds_contents(case):
    make = _cases()[case]
    say(f"[poison] {case}")
    nan_fill, call = make()
    torch.cuda.synchronize()
    q8 = _q8()
    first = None
    for p in PATTERNS:
        for t in nan_fill:
            t.fill_(float("nan") if t.is_floating_point() else 0xAB)
        q8.q8_0_debug_poison_lds(p)
        got = [t.clone() for t in call()]
        torch.cuda.synchronize()
        raw = [g.view(torch.uint8) if g.dtype != torch.uint8 else g for g in got]
        if first is None:
            first = raw
            for g in got:
                if g.dtype == torch.float32:
                    assert not torch.isnan(g).all(), f"{case}: output never written"
            continue
        for i, (a, b) in enumerate(zip(first, raw)):
            diff = (a != b).sum().item()
            assert diff == 0, f"{case}: output {i} differs in {diff} bytes after LDS pattern {p:#010x}"
