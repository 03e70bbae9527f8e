"""GPU parity: q8_0_quantize_act must equal the oracle's quantizer byte for byte."""
import numpy as np
import pytest
import torch

import workloads
from tests.helpers import cpu_u8, oracle_quantize, say

pytestmark = pytest.mark.gpu


def _q8():
    import q8_quantized_matmul_amd as q8
    return q8


def _check(x: torch.Tensor, where: str):
    q8 = _q8()
    say(f"[quantize] {where} shape={tuple(x.shape)}")
    got = q8.q8_0_quantize_act(x.cuda().contiguous())
    torch.cuda.synchronize()
    ref = oracle_quantize(x)
    g = cpu_u8(got)
    if not np.array_equal(g, ref):
        diff = np.argwhere(g != ref)
        raise AssertionError(f"{where}: {len(diff)} bytes differ, first at {diff[:4].tolist()}")


@pytest.mark.parametrize("n_tok,in_dim", [(1, 32), (3, 96), (5, 1024), (7, 4160), (64, 4096),
                                          (33, 2048), (2, 32768), (2000, 2112)])
def test_quantize_random_shapes(n_tok, in_dim):
    x = workloads.normal((n_tok, in_dim), 1.0, "cuda", "test_quantize", n_tok, in_dim)
    _check(x, f"randn {n_tok}x{in_dim}")


def test_quantize_special_values():
    x = torch.zeros((8, 256), dtype=torch.float32)
    d = 2.0 ** -5
    x[0, 0] = 127 * d
    x[0, 1:64] = torch.tensor([(k + 0.5) * d for k in range(-31, 32)], dtype=torch.float32)
    x[1, 5] = float("nan")
    x[1, 40] = float("inf")
    x[1, 70] = -float("inf")
    x[2, :32] = 8321040.0          # scale overflows binary16 -> marker
    x[2, 32:64] = 8319008.0        # max finite binary16 scale
    x[3, :32] = 2.0 ** -149        # fp32 scale underflows -> zero block
    x[3, 32] = 190 * 2.0 ** -149   # subnormal scale, clamp
    x[3, 64] = 127 * 2.0 ** -26    # binary16 scale rounds to zero
    x[3, 96] = 127 * 2.0 ** -20    # subnormal binary16 scale
    x[3, 97] = 2.0 ** -21
    x[4] = workloads.normal((256,), 1e-6, "cpu", "tiny_vals")
    x[5] = workloads.normal((256,), 3e4, "cpu", "huge_vals")
    x[6, ::2] = -0.0
    x[7] = workloads.normal((256,), 1.0, "cpu", "neg")
    x[7, 100] *= 50
    _check(x, "special values")


def test_quantize_near_ties():
    # Quotients one ulp either side of exact half-integers, with scales that are
    # not powers of two: the rounding decision depends on the IEEE quotient.
    rows = []
    for amax in (100.0, 3.3, 0.07, 777.7, 1e-3):
        d = np.float32(np.float32(amax) / np.float32(127.0))
        for start in range(-63, 63, 30):
            x = np.zeros(32, dtype=np.float32)
            x[0] = amax
            for i, k in enumerate(range(start, start + 30)):
                t = np.float32((k + 0.5) * np.float64(d))
                x[1 + i] = np.nextafter(t, np.float32(np.inf if i % 3 == 0 else -np.inf)) if i % 3 else t
            x[31] = -x[5]
            rows.append(x)
    _check(torch.from_numpy(np.stack(rows)), "near ties")


def test_quantize_near_ties_large():
    # The near-tie blocks tiled over more than 65536 block pairs (the launch
    # then gives each lane group four pairs), with a ragged last workgroup.
    rows = []
    for amax in (100.0, 3.3, 0.07, 777.7, 1e-3):
        d = np.float32(np.float32(amax) / np.float32(127.0))
        for start in range(-63, 63, 30):
            x = np.zeros(32, dtype=np.float32)
            x[0] = amax
            for i, k in enumerate(range(start, start + 30)):
                x[1 + i] = np.float32((k + 0.5) * np.float64(d))
                if i % 3:
                    x[1 + i] = np.nextafter(x[1 + i], np.float32(np.inf if i % 3 == 1 else -np.inf))
            x[31] = -x[5]
            rows.append(x)
    blocks = np.stack(rows)                                # 25 blocks of 32
    n_rows, row_blocks = 1990, 66                          # 65670 pairs, 65670 % 64 = 6
    tiled = np.resize(blocks, (n_rows * row_blocks, 32)).reshape(n_rows, row_blocks * 32)
    _check(torch.from_numpy(np.ascontiguousarray(tiled)), "near ties, four pairs per lane group")


@pytest.mark.parametrize("cfg", ["tiny", "attn_q_b", "decode5", "moe", "prefill_a", "prefill_b"])
def test_quantize_workloads(cfg):
    if cfg == "tiny":
        xs = [workloads.tiny("cuda")["x"], workloads.tiny("cuda")["w"]]
    elif cfg == "attn_q_b":
        xs = [workloads.attn_q_b("cuda")["x"]]
    elif cfg == "decode5":
        xs = [p["x"] for p in workloads.decode5("cuda")]
    elif cfg == "moe":
        xs = list(workloads.moe_acts("cuda"))
    else:
        xs = [workloads.prefill(cfg, "cuda")["x"]]
    for i, x in enumerate(xs):
        _check(x, f"{cfg}[{i}]")


def test_quantize_unaligned_fallback():
    q8 = _q8()
    x = workloads.normal((3, 96), 1.0, "cuda", "unaligned")
    buf = torch.full((3 * 102 + 2,), 0xAB, dtype=torch.uint8, device="cuda")
    view = buf[2:]                                   # 2-byte aligned only
    q8.q8_0_quantize_act(x, out=view)
    torch.cuda.synchronize()
    assert np.array_equal(cpu_u8(view).reshape(3, 102), oracle_quantize(x))
    assert cpu_u8(buf[:2]).tolist() == [0xAB, 0xAB]


def test_quantize_deterministic_and_sign_symmetric():
    q8 = _q8()
    x = workloads.normal((16, 2048), 1.0, "cuda", "det")
    a = cpu_u8(q8.q8_0_quantize_act(x))
    b = cpu_u8(q8.q8_0_quantize_act(x))
    c = cpu_u8(q8.q8_0_quantize_act(-x))
    torch.cuda.synchronize()
    assert np.array_equal(a, b)
    ab = a.reshape(16, 64, 34)
    cb = c.reshape(16, 64, 34)
    assert np.array_equal(ab[:, :, :2], cb[:, :, :2])
    assert np.array_equal(ab[:, :, 2:].view(np.int8), -cb[:, :, 2:].view(np.int8))
