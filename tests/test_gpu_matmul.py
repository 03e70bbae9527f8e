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
    ws = q8.matmul_workspace(in_dim, out_dim, n_tok, variant=variant, split_k=split)
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


@pytest.mark.parametrize("out_dim", [1, 67, 300])
@pytest.mark.parametrize("in_dim", [256, 512, 2048, 8192, 32768])
def test_single_token_staged_weights(in_dim, out_dim):
    # Single-token launches with rows of >= 4 pairs take their weights through
    # coalesced loads and a per-wave LDS transpose; regions that reach past
    # the last row are clamped to the matrix's end.  Out_dims that end inside
    # a region, every row-chunk layout (4 and 32 pairs per row, 64-pair chunks
    # over 2 and 4 waves, two chunks per wave), block sums and outputs.
    w = workloads.normal((out_dim, in_dim), 0.02, "cuda", "st1", out_dim, in_dim, "w")
    x = workloads.normal((1, in_dim), 1.0, "cuda", "st1", out_dim, in_dim, "x")
    wq, xq, wq_o, xq_o = _prep(w, x)
    _run_and_check(wq, xq, wq_o, xq_o, in_dim, out_dim, 1, 2, where="single-token matvec")
    q8 = _q8()
    got = q8.q8_0_matmul(wq, xq, in_dim, out_dim, 1)
    torch.cuda.synchronize()
    ref, mag, _ = oracle.matmul(wq_o, xq_o, in_dim)
    assert_close(got.cpu().numpy(), ref, mag, "single-token auto plan")


@pytest.mark.parametrize("n_tok", [1, 2, 5, 17, 33])
@pytest.mark.parametrize("in_dim", [256, 1024, 4096, 16384])
def test_matvec_token_counts(in_dim, n_tok):
    # From two tokens up the x rows go through LDS a bounded number at a time
    # (16 rows of 256 or 1024 values, 4 of 4096, 1 of 16384): these counts
    # cross those boundaries.
    out_dim = 45
    w = workloads.normal((out_dim, in_dim), 0.02, "cuda", "mvt", in_dim, "w")
    x = workloads.normal((n_tok, in_dim), 1.0, "cuda", "mvt", in_dim, n_tok, "x")
    wq, xq, wq_o, xq_o = _prep(w, x)
    got = _run_and_check(wq, xq, wq_o, xq_o, in_dim, out_dim, n_tok, 2, where="matvec tokens")
    # The product entry point (no block sums) on the same inputs.
    q8 = _q8()
    if q8.q8_0_matmul_plan(in_dim, out_dim, n_tok, 0)[0] == 2:
        prod = q8.q8_0_matmul(wq, xq, in_dim, out_dim, n_tok,
                              workspace=torch.empty(1, dtype=torch.uint8, device="cuda"))
        torch.cuda.synchronize()
        assert torch.equal(prod.view(torch.int32), got.view(torch.int32))


def _run_skinny(wq, xq, wq_o, xq_o, in_dim, out_dim, n_tok, split, where):
    # The skinny kernel's debug instantiation: outputs to tolerance and every
    # block's S_b bit-exactly; then the same call without block sums (the
    # product instantiation) must give the same outputs bit for bit.
    q8 = _q8()
    say(f"[matmul] {where} in={in_dim} out={out_dim} n_tok={n_tok} skinny split={split}")
    out = torch.full((n_tok, out_dim), float("nan"), device="cuda")
    ws = q8.matmul_workspace(in_dim, out_dim, n_tok, variant=q8.KERNEL_SKINNY, split_k=split)
    got, bs = q8.q8_0_matmul_debug(wq, xq, in_dim, out_dim, n_tok, variant=q8.KERNEL_SKINNY,
                                   split_k=split, blocksums=True, out=out, workspace=ws)
    plain, _ = q8.q8_0_matmul_debug(wq, xq, in_dim, out_dim, n_tok, variant=q8.KERNEL_SKINNY,
                                    split_k=split, blocksums=False, workspace=ws)
    torch.cuda.synchronize()
    assert not ws[:4096].any(), f"{where}: split-K arrival counters not re-armed"
    ref, mag, rbs = oracle.matmul(wq_o, xq_o, in_dim, want_blocksums=True)
    assert np.array_equal(bs.cpu().numpy(), rbs), f"{where}: block sums differ"
    assert torch.equal(plain.view(torch.int32), got.view(torch.int32)), f"{where}: debug build differs"
    got = got.cpu().numpy()
    assert_close(got, ref, mag, where)
    return got, ref


@pytest.mark.parametrize("in_dim,out_dim,n_tok,split", [
    (4096, 2048, 64, 4), (4096, 2048, 32, 4), (2048, 4096, 33, 2), (4096, 1000, 40, 1),
    (1024, 300, 17, 2), (64, 50, 64, 1), (192, 65, 31, 1), (128, 33, 5, 1), (4096, 64, 48, 16),
    (1024, 32768, 64, 1), (8192, 96, 1, 3), (2048, 4096, 64, 2), (4096, 2048, 64, 0),
    (16384, 2048, 64, 4), (4160, 2048, 64, 4), (4160, 300, 20, 3), (1024, 32768, 64, 2),
    (2048, 4096, 64, 1), (2048, 4096, 33, 1), (4096, 2050, 40, 1), (4160, 2048, 63, 1),
    (4096, 2048, 65, 1), (2048, 2048, 96, 0), (4160, 1000, 130, 0), (1024, 2050, 256, 0),
    (8192, 512, 200, 0), (192, 70, 129, 0), (16384, 520, 65, 0), (8192, 300, 130, 3),
    (4160, 100, 250, 2), (2048, 4096, 65, 0), (4096, 2048, 200, 1), (4096, 520, 40, 0)])
def test_skinny_shapes(in_dim, out_dim, n_tok, split):
    # Ragged rows and token counts, one or two token tiles, waves with no
    # block pair (192 values = 3 pairs), and split-K with uneven splits; K
    # ranges longer than the resident stages (16384, 8192), dword copies
    # (4160 values: 65 pairs) with split-K, and a split over 1024 tiles.
    # One split from 33 tokens with 64 to 128 row tiles puts the token tiles
    # in separate workgroups: a second tile of one token, ragged rows (65
    # row tiles) and dword copies.  Above 64 tokens (up to 256) every token
    # tile does: one token in the last tile, ragged rows and tokens, dword
    # copies, the longest rows the plan gives it (128 pairs), and K splits
    # there (partials and counters per row and token tile: the plan's two
    # splits for long rows, forced uneven splits, dword copies), and two
    # token tiles per workgroup where the grid is large (one token, then
    # eight, in the last workgroup).  From 33 tokens, rows of up to 64 pairs
    # also split their token tiles beside a K split (4096 -> 520 at 40).
    w = workloads.normal((out_dim, in_dim), 0.02, "cuda", "sk", out_dim, in_dim, "w")
    x = workloads.normal((n_tok, in_dim), 1.0, "cuda", "sk", n_tok, in_dim, "x")
    x[min(3, n_tok - 1), 40:50] *= 30.0  # outlier block
    wq, xq, wq_o, xq_o = _prep(w, x)
    _run_skinny(wq, xq, wq_o, xq_o, in_dim, out_dim, n_tok, split, "skinny")


def test_skinny_workspace_reuse_and_graph():
    """One zero-filled workspace serves calls of different shapes and splits:
    the in-launch split-K arrival counters are back at zero after every call,
    so later calls and graph replays find them armed."""
    q8 = _q8()
    # Above 64 tokens a split keeps one counter per (row tile, token tile).
    shapes = [(4096, 2048, 64, 4), (2048, 256, 20, 8), (16384, 520, 100, 2), (4160, 2048, 64, 4),
              (4096, 2048, 64, 4), (16384, 520, 100, 2)]
    need = max(q8.q8_0_matmul_debug_workspace_bytes(k, n, t, q8.KERNEL_SKINNY, sp)
               for k, n, t, sp in shapes)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    data, firsts = {}, {}
    for k, n, t, sp in shapes:
        if (k, n, t) not in data:
            w = workloads.normal((n, k), 0.02, "cuda", "skr", n, k, "w")
            x = workloads.normal((t, k), 1.0, "cuda", "skr", t, k, "x")
            data[(k, n, t)] = _prep(w, x)
        wq, xq, wq_o, xq_o = data[(k, n, t)]
        say(f"[matmul] skinny reuse in={k} out={n} n_tok={t} split={sp}")
        out = torch.full((t, n), float("nan"), device="cuda")
        q8.q8_0_matmul_debug(wq, xq, k, n, t, variant=q8.KERNEL_SKINNY, split_k=sp,
                             blocksums=False, out=out, workspace=ws)
        torch.cuda.synchronize()
        assert not ws[:4096].any(), "arrival counters not re-armed"
        ref, mag, _ = oracle.matmul(wq_o, xq_o, k)
        assert_close(out.cpu().numpy(), ref, mag, f"skinny reuse {k}x{n}x{t}")
        if (k, n, t) in firsts:
            assert torch.equal(out.view(torch.int32), firsts[(k, n, t)].view(torch.int32))
        firsts[(k, n, t)] = out
    # Graph capture of split-K calls; every replay equals the eager result.
    for k, n, t, sp in (shapes[0], shapes[2]):
        wq, xq, _, _ = data[(k, n, t)]
        out = torch.empty((t, n), device="cuda")
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                q8.q8_0_matmul_debug(wq, xq, k, n, t, variant=q8.KERNEL_SKINNY, split_k=sp,
                                     blocksums=False, out=out, workspace=ws)
        torch.cuda.current_stream().wait_stream(s)
        for rep in range(3):
            out.fill_(float("nan"))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int32), firsts[(k, n, t)].view(torch.int32)), rep
            assert not ws[:4096].any()


@pytest.mark.parametrize("only_block", [None, 0, 1, 2, 3, 6, 7])
@pytest.mark.parametrize("n_tok", [64, 20])
def test_skinny_exact_integer_sums(only_block, n_tok):
    # Unit scales: every output is the exact integer sum of the block dots
    # (below 2^24), and with one nonzero block it is that block's S_b; this
    # pins both halves of the even (re-aligned) and odd blocks of a pair, in
    # every wave and across two splits.
    in_dim, out_dim = 512, 96
    nb = in_dim // 32
    w_b = _unit_scale_blocks(out_dim, nb, 21, only_block)
    x_b = _unit_scale_blocks(n_tok, nb, 22, only_block)
    wq = torch.from_numpy(w_b).cuda()
    xq = torch.from_numpy(x_b).cuda()
    got, ref = _run_skinny(wq, xq, w_b, x_b, in_dim, out_dim, n_tok, 2,
                           f"skinny unit scales block={only_block}")
    _, _, bs = oracle.matmul(w_b, x_b, in_dim, want_blocksums=True)
    exact = bs.astype(np.int64).sum(axis=2)
    assert np.abs(exact).max() < 2 ** 24
    assert np.array_equal(got.astype(np.float64), exact.astype(np.float64))
    assert np.array_equal(ref.astype(np.float64), exact.astype(np.float64))


def test_skinny_special_scales():
    # Subnormal weight scales, a NaN activation, a zero block.
    in_dim, out_dim, n_tok = 512, 70, 40
    w = workloads.normal((out_dim, in_dim), 2e-7, "cuda", "sksub", "w")
    x = workloads.normal((n_tok, in_dim), 1.0, "cuda", "sksub", "x")
    x[3, 17] = float("nan")
    x[30, 64:96] = 0.0
    wq, xq, wq_o, xq_o = _prep(w, x)
    _run_skinny(wq, xq, wq_o, xq_o, in_dim, out_dim, n_tok, 2, "skinny special")


@pytest.mark.parametrize("in_dim", [32, 96, 160, 3072, 4160])
def test_generic_only_shapes(in_dim):
    q8 = _q8()
    out_dim, n_tok = 19, 2
    w = workloads.normal((out_dim, in_dim), 0.02, "cuda", "gen", in_dim, "w")
    x = workloads.normal((n_tok, in_dim), 1.0, "cuda", "gen", in_dim, "x")
    wq, xq, wq_o, xq_o = _prep(w, x)
    # Rows the matvec cannot take: the generic kernel, or from two tokens the
    # skinny kernel where rows are whole block pairs (3072, 4160).
    assert q8.q8_0_matmul_plan(in_dim, out_dim, n_tok, 0)[0] == (4 if in_dim % 64 == 0 else 1)
    _run_and_check(wq, xq, wq_o, xq_o, in_dim, out_dim, n_tok, 0, where="auto")


@pytest.mark.parametrize("out_dim,n_tok,in_dim,split", [
    (300, 150, 1152, 1), (300, 150, 1152, 3), (128, 64, 4096, 1), (77, 16, 2048, 4),
    (256, 257, 512, 2), (33, 1, 1024, 1), (130, 70, 8192, 16)])
def test_mfma_ragged(out_dim, n_tok, in_dim, split):
    w = workloads.normal((out_dim, in_dim), 0.02, "cuda", "mf", out_dim, in_dim, "w")
    x = workloads.normal((n_tok, in_dim), 1.0, "cuda", "mf", n_tok, in_dim, "x")
    wq, xq, wq_o, xq_o = _prep(w, x)
    _run_and_check(wq, xq, wq_o, xq_o, in_dim, out_dim, n_tok, 3, split, where="mfma")


def _run_outputs(wq, xq, wq_o, xq_o, in_dim, out_dim, n_tok, split, where):
    """MFMA path without block sums (whole-tile shapes then take the four-tile
    kernel, which has no block-sum output): outputs against the oracle."""
    q8 = _q8()
    say(f"[matmul] {where} in={in_dim} out={out_dim} n_tok={n_tok} split={split}")
    out = torch.full((n_tok, out_dim), float("nan"), device="cuda")
    ws = q8.matmul_workspace(in_dim, out_dim, n_tok, variant=3, split_k=split)
    got, _ = q8.q8_0_matmul_debug(wq, xq, in_dim, out_dim, n_tok, variant=3, split_k=split,
                                  blocksums=False, out=out, workspace=ws)
    torch.cuda.synchronize()
    ref, mag, _ = oracle.matmul(wq_o, xq_o, in_dim)
    assert_close(got.cpu().numpy(), ref, mag, where)
    return got.cpu().numpy(), ref


def _at_offset(t, off):
    """A copy of uint8 tensor t whose data starts `off` bytes into a larger buffer."""
    buf = torch.zeros(t.numel() + 64, dtype=torch.uint8, device=t.device)
    v = buf[off:off + t.numel()].view(t.shape)
    v.copy_(t)
    return v


@pytest.mark.parametrize("out_dim,n_tok,in_dim", [
    (256, 256, 512),     # whole tiles: the four-tile kernel when 16-byte aligned
    (300, 150, 1152),    # ragged: the direct-copy tiled kernel when aligned
    (512, 40, 1024),     # the skinny kernel (16-byte or dword copies)
    (1024, 1, 32768),    # single-token matvec, coalesced x chunks
    (1024, 5, 4096)])    # several tokens, staged x rows
def test_operands_at_4_byte_offsets(out_dim, n_tok, in_dim):
    # w and x_q 4 bytes into larger buffers: the kernels that copy 16-byte
    # chunks must not take them.  The auto plan's result is checked against
    # the oracle, and against the same call on the aligned copies.
    q8 = _q8()
    w = workloads.normal((out_dim, in_dim), 0.02, "cuda", "off4", out_dim, in_dim, "w")
    x = workloads.normal((n_tok, in_dim), 1.0, "cuda", "off4", n_tok, in_dim, "x")
    wq, xq, wq_o, xq_o = _prep(w, x)
    wq4, xq4 = _at_offset(wq, 4), _at_offset(xq, 4)
    assert wq4.data_ptr() % 16 == 4 and xq4.data_ptr() % 16 == 4
    say(f"[matmul] offset4 in={in_dim} out={out_dim} n_tok={n_tok}")
    got = q8.q8_0_matmul(wq4, xq4, in_dim, out_dim, n_tok)
    aligned = q8.q8_0_matmul(wq, xq, in_dim, out_dim, n_tok)
    torch.cuda.synchronize()
    ref, mag, _ = oracle.matmul(wq_o, xq_o, in_dim)
    assert_close(got.cpu().numpy(), ref, mag, f"offset4 {out_dim}x{n_tok}x{in_dim}")
    assert_close(aligned.cpu().numpy(), ref, mag, f"aligned {out_dim}x{n_tok}x{in_dim}")


@pytest.mark.parametrize("out_dim,n_tok,in_dim,split", [
    (256, 256, 512, 1), (384, 128, 1152, 3), (128, 384, 4096, 1), (256, 128, 2048, 4),
    (512, 128, 128, 1), (768, 256, 384, 1), (1024, 128, 640, 1), (256, 256, 1024, 2)])
def test_mfma_whole_tiles(out_dim, n_tok, in_dim, split):
    # Whole 128 x 128 tiles with 4-block stages: the four-tile kernel, with
    # one to five stages per split, also with split-K.
    w = workloads.normal((out_dim, in_dim), 0.02, "cuda", "mf4", out_dim, in_dim, "w")
    x = workloads.normal((n_tok, in_dim), 1.0, "cuda", "mf4", n_tok, in_dim, "x")
    x[5, 100:110] *= 40.0  # outlier block
    wq, xq, wq_o, xq_o = _prep(w, x)
    _run_outputs(wq, xq, wq_o, xq_o, in_dim, out_dim, n_tok, split, "mfma4")


def test_mfma_whole_tiles_special_scales():
    in_dim, out_dim, n_tok = 512, 128, 128
    w = workloads.normal((out_dim, in_dim), 2e-7, "cuda", "sub4", "w")
    x = workloads.normal((n_tok, in_dim), 1.0, "cuda", "sub4", "x")
    x[3, 17] = float("nan")
    x[70, 64:96] = 0.0
    wq, xq, wq_o, xq_o = _prep(w, x)
    _run_outputs(wq, xq, wq_o, xq_o, in_dim, out_dim, n_tok, 1, "mfma4 special")


def _unit_scale_blocks(rows, nb, seed, only_block=None):
    """Q8_0 bytes with every scale binary16 1.0 and uniform int8 quants in
    [-127, 127] (all quants zero outside `only_block` when it is given)."""
    rng = np.random.default_rng(seed)
    q = rng.integers(-127, 128, size=(rows, nb, 32), dtype=np.int64).astype(np.int8)
    if only_block is not None:
        keep = np.zeros(nb, dtype=bool)
        keep[only_block] = True
        q[:, ~keep, :] = 0
    blk = np.zeros((rows, nb, 34), dtype=np.uint8)
    blk[:, :, 0] = 0x00
    blk[:, :, 1] = 0x3C  # binary16 1.0, little-endian
    blk[:, :, 2:] = q.view(np.uint8)
    return blk.reshape(rows, nb * 34)


@pytest.mark.parametrize("only_block", [None, 0, 1, 2, 3, 5, 14])
@pytest.mark.parametrize("split", [1, 2])
@pytest.mark.parametrize("out_dim", [256, 128])
def test_mfma_whole_tiles_exact_integer_sums(only_block, split, out_dim):
    # With unit scales every term is an integer and every partial sum stays
    # below 2^24, so the fp32 output must equal the exact sum of the block
    # dots; with one nonzero block it is that block's S_b.  This pins the
    # integer path of the four-tile kernel (which has no block-sum output)
    # bit-exactly, block by block across stage positions and stages.
    in_dim, n_tok = 512, 128
    nb = in_dim // 32
    w_b = _unit_scale_blocks(out_dim, nb, 11, only_block)
    x_b = _unit_scale_blocks(n_tok, nb, 12, only_block)
    wq = torch.from_numpy(w_b).cuda()
    xq = torch.from_numpy(x_b).cuda()
    got, ref = _run_outputs(wq, xq, w_b, x_b, in_dim, out_dim, n_tok, split,
                            f"mfma4 unit scales block={only_block}")
    _, _, bs = oracle.matmul(w_b, x_b, in_dim, want_blocksums=True)
    exact = bs.astype(np.int64).sum(axis=2)
    assert np.abs(exact).max() < 2 ** 24
    assert np.array_equal(got.astype(np.float64), exact.astype(np.float64))
    assert np.array_equal(ref.astype(np.float64), exact.astype(np.float64))


def test_mfma_whole_tiles_extreme_block_sums():
    # Block sums at the ends of their range, |S_b| = 32 * 127 * 127 = 516128,
    # of both signs, next to sums of 0 and +-1: the four-tile kernel turns
    # each block's int32 sum into fp32 on the matrix core (a biased
    # accumulator and an exact unbias), which must stay exact across the
    # whole range.  Unit scales keep every output an exact integer < 2^24.
    in_dim, out_dim, n_tok = 512, 128, 128
    nb = in_dim // 32
    rng = np.random.default_rng(21)
    qw = np.full((out_dim, nb, 32), 127, dtype=np.int64)
    qw[::3] = -127                                   # rows of -127 as well
    sign = rng.choice([-1, 1], size=(n_tok, nb, 1))
    qx = np.broadcast_to(127 * sign, (n_tok, nb, 32)).copy()
    qx[::5, :, :] = 0                                # S_b = 0
    qx[1::5, :, :] = 0
    qx[1::5, :, 0] = 1                               # S_b = +-127
    qx[2::5, :, 1:] = 0
    qx[2::5, :, 0] = -1                              # S_b = -+127

    def blocks(q):
        b = np.zeros(q.shape[:2] + (34,), dtype=np.uint8)
        b[:, :, 1] = 0x3C                            # binary16 1.0
        b[:, :, 2:] = q.astype(np.int8).view(np.uint8)
        return b.reshape(q.shape[0], -1)

    w_b, x_b = blocks(qw), blocks(qx)
    got, ref = _run_outputs(torch.from_numpy(w_b).cuda(), torch.from_numpy(x_b).cuda(),
                            w_b, x_b, in_dim, out_dim, n_tok, 1, "mfma4 extreme sums")
    exact = np.einsum("tbk,obk->to", qx, qw)
    assert np.abs(exact).max() < 2 ** 24
    assert np.array_equal(got.astype(np.float64), exact.astype(np.float64))


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
def test_prefill_full(name):
    """Full-size launch as timed by the benchmark (the automatic plan, its
    split-K workspace): every quantized weight and activation byte and every
    output element against the oracle (on the host's cores)."""
    q8 = _q8()
    d = workloads.prefill(name, "cuda")
    k, n, t = d["in_dim"], d["out_dim"], d["n_tok"]
    wq = q8.q8_0_quantize_act(d["w"])
    xq = q8.q8_0_quantize_act(d["x"])
    ws = q8.matmul_workspace(k, n, t)
    plan = q8.q8_0_matmul_plan(k, n, t, ws.numel())
    say(f"[matmul] {name} full plan={plan}")
    assert plan[0] == q8.KERNEL_MFMA
    out = torch.full((t, n), float("nan"), device="cuda")
    got = q8.q8_0_matmul(wq, xq, k, n, t, out=out, workspace=ws)
    torch.cuda.synchronize()
    with oracle.threads():
        xq_o = oracle_quantize(d["x"])
        wq_o = oracle_quantize(d["w"])
        assert np.array_equal(cpu_u8(xq), xq_o)
        assert np.array_equal(cpu_u8(wq), wq_o)
        say(f"[matmul] {name} oracle on {oracle.get_threads()} threads")
        ref, mag, _ = oracle.matmul(wq_o, xq_o, k)
    assert_close(got.cpu().numpy(), ref, mag, name)


@pytest.mark.parametrize("name,rows,tokens,split", [
    ("prefill_a", 256, 256, 1), ("prefill_a", 128, 384, 2), ("prefill_b", 128, 256, 0)])
def test_prefill_whole_tile_blocksums(name, rows, tokens, split):
    # Whole 128 x 128 tiles of each prefill workload (whole K), so the call
    # runs the four-tile kernel the benchmark times, in its debug
    # instantiation: every block's S_b bit-exactly and the outputs, which must
    # equal the product instantiation's bit for bit.
    q8 = _q8()
    d = workloads.prefill(name, "cuda", rows=rows, tokens=tokens)
    wq, xq, wq_o, xq_o = _prep(d["w"], d["x"])
    k = d["in_dim"]
    got = _run_and_check(wq, xq, wq_o, xq_o, k, rows, tokens, q8.KERNEL_MFMA, split,
                         where=f"{name} whole tiles")
    ws = q8.matmul_workspace(k, rows, tokens, variant=q8.KERNEL_MFMA, split_k=split)
    plain, _ = q8.q8_0_matmul_debug(wq, xq, k, rows, tokens, variant=q8.KERNEL_MFMA, split_k=split,
                                    blocksums=False, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(plain.view(torch.int32), got.view(torch.int32))


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


def _random_shapes(n_cases, seed):
    """Seeded shapes around the plan's regime edges (1-2 tokens, 15-21, 60-70,
    above 100), in_dim any multiple of 32 up to 8192, ragged out_dim; the
    oracle's work per case is bounded."""
    rng = np.random.default_rng(seed)
    tok_pool = [1, 2, 3, 15, 16, 17, 19, 20, 21, 33, 63, 64, 65, 66, 70, 97, 128, 129, 160]
    cases = []
    while len(cases) < n_cases:
        kind = rng.integers(0, 3)
        if kind == 0:
            in_dim = 32 * int(rng.integers(1, 257))
        elif kind == 1:
            in_dim = 64 * 2 ** int(rng.integers(0, 8))
        else:
            in_dim = 4096 * int(rng.integers(1, 3))
        out_dim = int(rng.integers(1, 2500))
        n_tok = int(rng.choice(tok_pool))
        if in_dim * out_dim * n_tok <= 1.5e8:
            cases.append((in_dim, out_dim, n_tok))
    return cases


@pytest.mark.parametrize("in_dim,out_dim,n_tok", _random_shapes(36, 2024))
def test_auto_plan_random_shapes(in_dim, out_dim, n_tok):
    # Whatever kernel and split the plan picks for the shape (with the
    # workspace it asks for) matches the oracle; the output starts poisoned.
    q8 = _q8()
    w = workloads.normal((out_dim, in_dim), 0.02, "cuda", "rand", in_dim, out_dim, "w")
    x = workloads.normal((n_tok, in_dim), 1.0, "cuda", "rand", in_dim, n_tok, "x")
    wq, xq, wq_o, xq_o = _prep(w, x)
    ws = q8.matmul_workspace(in_dim, out_dim, n_tok)
    plan = q8.q8_0_matmul_plan(in_dim, out_dim, n_tok, ws.numel())
    say(f"[matmul random] in={in_dim} out={out_dim} n_tok={n_tok} plan={plan}")
    out = torch.full((n_tok, out_dim), float("nan"), device="cuda")
    got = q8.q8_0_matmul(wq, xq, in_dim, out_dim, n_tok, out=out, workspace=ws)
    torch.cuda.synchronize()
    ref, mag, _ = oracle.matmul(wq_o, xq_o, in_dim)
    assert_close(got.cpu().numpy(), ref, mag, f"random {in_dim}x{out_dim}x{n_tok} plan {plan}")
