"""CPU checks of the C ABI: the library loads, exports every function that
include/q8_0.h declares, and its host-side argument checks and kernel plan
behave as documented.  No compute call reaches a device here: every call
either fails validation before any HIP call, or is host-only."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "q8_0.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(q8_0_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def q8():
    import q8_quantized_matmul_amd as m
    return m


def test_exports_every_declared_symbol(q8):
    lib = ctypes.CDLL(q8.LIB_PATH)
    declared = _declared()
    assert len(declared) == 20
    for name in declared:
        assert hasattr(lib, name), name
    assert set(declared) == set(q8.EXPORTED)


def _prototype(name):
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    m = re.search(r"\b(\w[\w\s\*]*?)\b" + name + r"\s*\(([^;]*?)\)\s*;", text, flags=re.S)
    assert m, name
    ret = " ".join(m.group(1).split())
    params = [" ".join(p.split()) for p in m.group(2).split(",")]
    return ret, params


def test_boundary_signatures():
    """The three calls of the path and their departures from the plain
    (out, w, in_dim, out_dim, x, n_tok) form: caller workspace for split-K,
    a device expert table, and a workspace size without out_dim."""
    assert _prototype("q8_0_quantize_act") == (
        "int", ["void *x_q", "const float *x", "int64_t n_tok", "int64_t in_dim",
                "hipStream_t stream"])
    assert _prototype("q8_0_matmul") == (
        "int", ["float *out", "const void *w", "int64_t in_dim", "int64_t out_dim",
                "const void *x_q", "int64_t n_tok", "void *workspace", "size_t workspace_bytes",
                "hipStream_t stream"])
    assert _prototype("q8_0_moe_grouped") == (
        "int", ["float *out", "const void *const *expert_w", "int32_t n_expert",
                "int64_t in_dim", "int64_t out_dim", "const int32_t *selected",
                "int32_t n_used", "const void *x_q", "int32_t x_rows", "int64_t n_tok",
                "void *workspace", "size_t workspace_bytes", "hipStream_t stream"])
    assert _prototype("q8_0_moe_workspace_bytes") == (
        "size_t", ["int64_t n_tok", "int32_t n_used", "int32_t n_expert"])


def test_strerror(q8):
    assert q8.q8_0_strerror(0) == "ok"
    for code in (-1, -2, -3, -4, -5):
        assert q8.q8_0_strerror(code) != "unknown status"


FAKE = 0x10000  # never dereferenced: every call below fails validation first


def test_quantize_validation(q8):
    lib = q8.raw_library()
    assert lib.q8_0_quantize_act(FAKE, FAKE, 1, 33, None) == q8.Q8_0_EINVAL
    assert lib.q8_0_quantize_act(FAKE, FAKE, -1, 32, None) == q8.Q8_0_EINVAL
    assert lib.q8_0_quantize_act(None, FAKE, 1, 32, None) == q8.Q8_0_EINVAL
    assert lib.q8_0_quantize_act(FAKE + 1, FAKE, 1, 32, None) == q8.Q8_0_EALIGN
    assert lib.q8_0_quantize_act(FAKE, FAKE + 2, 1, 32, None) == q8.Q8_0_EALIGN
    assert lib.q8_0_quantize_act(FAKE, FAKE, 0, 32, None) == q8.Q8_0_OK  # empty


def test_matmul_validation(q8):
    lib = q8.raw_library()
    mm = lib.q8_0_matmul
    assert mm(FAKE, FAKE, 48, 4, FAKE, 1, None, 0, None) == q8.Q8_0_EINVAL
    assert mm(FAKE, FAKE, 0, 4, FAKE, 1, None, 0, None) == q8.Q8_0_EINVAL
    assert mm(FAKE, None, 32, 4, FAKE, 1, None, 0, None) == q8.Q8_0_EINVAL
    assert mm(FAKE + 2, FAKE, 32, 4, FAKE, 1, None, 0, None) == q8.Q8_0_EALIGN
    assert mm(FAKE, FAKE + 1, 32, 4, FAKE, 1, None, 0, None) == q8.Q8_0_EALIGN
    assert mm(FAKE, FAKE, 32, 0, FAKE, 1, None, 0, None) == q8.Q8_0_OK
    assert mm(None, None, 32, 4, None, 0, None, 0, None) == q8.Q8_0_OK
    dbg = lib.q8_0_matmul_debug
    # forced matvec on a shape without whole block pairs
    assert dbg(FAKE, None, FAKE, 96, 4, FAKE, 1, None, 0, 2, 0, None) == q8.Q8_0_EINVAL
    # forced MFMA on 2-byte aligned operands
    assert dbg(FAKE, None, FAKE + 2, 128, 4, FAKE, 32, None, 0, 3, 0, None) == q8.Q8_0_EINVAL
    # forced split without workspace
    assert dbg(FAKE, None, FAKE, 4096, 256, FAKE, 64, None, 0, 3, 4, None) == q8.Q8_0_EWORKSPACE
    # split on a non-MFMA variant
    assert dbg(FAKE, None, FAKE, 4096, 256, FAKE, 1, None, 0, 2, 2, None) == q8.Q8_0_EINVAL
    assert dbg(FAKE, None, FAKE, 4096, 256, FAKE, 1, None, 0, 7, 0, None) == q8.Q8_0_EINVAL


def test_moe_validation(q8):
    lib = q8.raw_library()
    mo = lib.q8_0_moe_grouped
    need = q8.q8_0_moe_workspace_bytes(64, 8, 256)
    assert need >= 4 * (16 + 2 * 256 + 1 + 512) and need % 256 == 0
    args = dict(n_expert=256, in_dim=4096, out_dim=2048, n_used=8, x_rows=0, n_tok=64)

    def call(**kw):
        a = dict(args, **kw)
        return mo(FAKE, FAKE, a["n_expert"], a["in_dim"], a["out_dim"], FAKE, a["n_used"], FAKE,
                  a["x_rows"], a["n_tok"], kw.get("ws", FAKE), kw.get("ws_bytes", need), None)

    assert call(n_expert=0) == q8.Q8_0_EINVAL
    assert call(n_expert=100000) == q8.Q8_0_EINVAL
    assert call(n_used=0) == q8.Q8_0_EINVAL
    assert call(x_rows=2) == q8.Q8_0_EINVAL
    assert call(in_dim=4100) == q8.Q8_0_EINVAL
    assert call(ws_bytes=need - 4) == q8.Q8_0_EWORKSPACE
    assert call(ws=None) == q8.Q8_0_EWORKSPACE
    assert call(n_tok=0) == q8.Q8_0_OK


def test_moe_noalloc_validation(q8):
    lib = q8.raw_library()
    mo = lib.q8_0_moe_grouped_noalloc
    assert q8.MOE_STATIC_SCRATCH_BYTES == 1 << 20

    def call(n_expert=256, in_dim=4096, out_dim=2048, n_used=8, x_rows=0, n_tok=64, inv=None,
             out=FAKE):
        return mo(out, FAKE, n_expert, in_dim, out_dim, FAKE, n_used, FAKE, x_rows, n_tok, inv,
                  None)

    assert call(n_expert=0) == q8.Q8_0_EINVAL
    assert call(n_used=0) == q8.Q8_0_EINVAL
    assert call(x_rows=2) == q8.Q8_0_EINVAL
    assert call(in_dim=4100) == q8.Q8_0_EINVAL
    assert call(out=FAKE + 2) == q8.Q8_0_EALIGN
    assert call(inv=FAKE + 2) == q8.Q8_0_EALIGN
    assert call(n_tok=0) == q8.Q8_0_OK
    # The largest routing shape the static tables hold, and one pair more.
    ints = q8.MOE_STATIC_SCRATCH_BYTES // 4 - (16 + 2 * 256 + 1)
    assert q8.q8_0_moe_workspace_bytes(ints, 1, 256) <= q8.MOE_STATIC_SCRATCH_BYTES
    assert call(n_tok=ints + 1, n_used=1) == q8.Q8_0_EWORKSPACE


def test_list_validation(q8):
    lib = q8.raw_library()

    def call(items, n_tok=1, n=None):
        arr = (q8.MatmulItem * max(len(items), 1))(*items)
        return lib.q8_0_matmul_list(arr, len(items) if n is None else n, n_tok, None)

    def item(out=FAKE, w=FAKE, x=None, x_q=FAKE, in_dim=1024, out_dim=256):
        return q8.MatmulItem(out, w, x, x_q, in_dim, out_dim)

    assert call([item()], n=0) == q8.Q8_0_EINVAL
    assert call([item()] * 17) == q8.Q8_0_EINVAL
    assert lib.q8_0_matmul_list(None, 1, 1, None) == q8.Q8_0_EINVAL
    assert call([item(), item(in_dim=1000)]) == q8.Q8_0_EINVAL
    assert call([item(out=None)]) == q8.Q8_0_EINVAL
    assert call([item(x=None, x_q=None)]) == q8.Q8_0_EINVAL
    assert call([item(out=FAKE + 2)]) == q8.Q8_0_EALIGN
    assert call([item(x=FAKE + 2, x_q=None)]) == q8.Q8_0_EALIGN
    assert call([item(), item()], n_tok=-1) == q8.Q8_0_EINVAL
    # x without x_q is only allowed where the launch quantizes x itself:
    # in_dim 64 * 2^k <= 4096 with n_tok * in_dim <= 4096, 16-byte aligned x.
    assert call([item(x=FAKE, x_q=None, in_dim=8192)]) == q8.Q8_0_EINVAL
    assert call([item(x=FAKE, x_q=None, in_dim=4096)], n_tok=2) == q8.Q8_0_EINVAL
    assert call([item(x=FAKE + 4, x_q=None, in_dim=1024)]) == q8.Q8_0_EINVAL
    assert call([item(x=FAKE, x_q=None, in_dim=96)]) == q8.Q8_0_EINVAL
    # empty work is a successful no-op
    assert call([item()], n_tok=0) == q8.Q8_0_OK
    assert call([item(out=None, w=None, x_q=None, out_dim=0)]) == q8.Q8_0_OK


def test_moe_ffn_validation(q8):
    lib = q8.raw_library()
    need = q8.q8_0_moe_ffn_workspace_bytes(64, 8, 256, 4096, 2048)
    pairs = 512
    assert need >= pairs * 2048 * 4 + pairs * 64 * 34 + pairs * 4096 * 4

    def call(ws=FAKE, ws_bytes=need, **kw):
        f = dict(out=FAKE, gate_w=FAKE, up_w=FAKE, down_w=FAKE, n_expert=256, n_used=8,
                 d_model=4096, d_ff=2048, n_tok=64, selected=FAKE, weights=FAKE, x_q=FAKE,
                 clamp=0.0, mid=None, mid_q=None, y=None)
        f.update(kw)
        a = q8.MoeFfnArgs(**f)
        return lib.q8_0_moe_ffn(ctypes.byref(a), ws, ws_bytes, None)

    assert lib.q8_0_moe_ffn(None, FAKE, need, None) == q8.Q8_0_EINVAL
    assert call(n_expert=0) == q8.Q8_0_EINVAL
    assert call(n_used=0) == q8.Q8_0_EINVAL
    assert call(d_model=4100) == q8.Q8_0_EINVAL
    assert call(d_model=12288) == q8.Q8_0_EINVAL      # 3 chunks per wave: no paired kernel
    assert call(d_ff=96) == q8.Q8_0_EINVAL
    assert call(weights=None) == q8.Q8_0_EINVAL
    assert call(mid=FAKE + 4) == q8.Q8_0_EALIGN
    assert call(ws_bytes=need - 1) == q8.Q8_0_EWORKSPACE
    assert call(ws=None) == q8.Q8_0_EWORKSPACE
    assert call(ws=FAKE + 16) == q8.Q8_0_EALIGN
    assert call(n_tok=0) == q8.Q8_0_OK


def test_plan_regimes(q8):
    # Decode shapes stream weights through the matvec kernel.
    assert q8.q8_0_matmul_plan(1024, 32768, 1, 0) == (q8.KERNEL_MATVEC, 1)
    assert q8.q8_0_matmul_plan(32768, 1024, 1, 0) == (q8.KERNEL_MATVEC, 1)
    assert q8.q8_0_matmul_plan(4096, 2048, 11, 0) == (q8.KERNEL_MATVEC, 1)
    assert q8.q8_0_matmul_plan(4096, 2048, 12, 0) == (q8.KERNEL_SKINNY, 1)
    # Rows the matvec cannot take: the generic kernel at one token, the
    # skinny kernel from two.
    assert q8.q8_0_matmul_plan(7168, 2048, 1, 0) == (q8.KERNEL_GENERIC, 1)
    assert q8.q8_0_matmul_plan(7168, 2048, 2, 0) == (q8.KERNEL_SKINNY, 1)
    assert q8.q8_0_matmul_plan(1536, 4096, 4, 1 << 40)[0] == q8.KERNEL_SKINNY
    # From 12 to 64 tokens the skinny matrix-core kernel.  Split-K only
    # below 128 tiles of 32 rows: about 256 workgroups, at least 16 block
    # pairs per split, at most 16 splits.
    assert q8.q8_0_matmul_plan(4096, 2048, 16, 1 << 40) == (q8.KERNEL_SKINNY, 4)
    # From 33 tokens with 64 to 128 row tiles the token tiles go to separate
    # workgroups instead: one split, no workspace.
    assert q8.q8_0_matmul_plan(4096, 2048, 64, 1 << 40) == (q8.KERNEL_SKINNY, 1)
    assert q8.q8_0_matmul_plan(4096, 2048, 32, 1 << 40) == (q8.KERNEL_SKINNY, 4)
    assert q8.q8_0_matmul_plan(4096, 1024, 33, 1 << 40) == (q8.KERNEL_SKINNY, 4)
    assert q8.q8_0_matmul_plan(4096, 2048, 64, 0) == (q8.KERNEL_SKINNY, 1)
    assert q8.q8_0_matmul_plan(2048, 4096, 16, 1 << 40) == (q8.KERNEL_SKINNY, 1)
    assert q8.q8_0_matmul_plan(2048, 4064, 16, 1 << 40) == (q8.KERNEL_SKINNY, 2)
    assert q8.q8_0_matmul_plan(1024, 32768, 64, 1 << 40) == (q8.KERNEL_SKINNY, 1)
    assert q8.q8_0_matmul_plan(4096, 1024, 64, 1 << 40) == (q8.KERNEL_SKINNY, 4)
    assert q8.q8_0_matmul_plan(7168, 2048, 32, 1 << 40) == (q8.KERNEL_SKINNY, 4)
    assert q8.q8_0_matmul_plan(4096, 256, 48, 1 << 40) == (q8.KERNEL_SKINNY, 4)
    assert q8.q8_0_matmul_plan(65536, 256, 20, 1 << 40) == (q8.KERNEL_SKINNY, 16)
    # Split-K workspace: 4096 bytes of arrival counters, then 4 KiB of
    # partials per 32-token tile for each workgroup (64 tiles x 4 splits).
    assert q8.q8_0_matmul_workspace_bytes(4096, 2048, 64) == 0
    assert q8.q8_0_matmul_workspace_bytes(4096, 1024, 64) == 4096 + 4 * 32 * 2 * 4096
    assert q8.q8_0_matmul_workspace_bytes(4096, 2048, 16) == 4096 + 4 * 64 * 1 * 4096
    assert q8.q8_0_matmul_debug_workspace_bytes(4096, 2048, 64, q8.KERNEL_SKINNY, 2) == \
        4096 + 2 * 64 * 2 * 4096
    assert q8.q8_0_matmul_debug_workspace_bytes(4096, 2048, 64, q8.KERNEL_SKINNY, 1) == 0
    # A skinny split needs one counter per 32-row tile: at most 1024 tiles.
    assert q8.q8_0_matmul_debug_workspace_bytes(1024, 32768, 64, q8.KERNEL_SKINNY, 2) > 0
    assert q8.q8_0_matmul_debug_workspace_bytes(1024, 32800, 64, q8.KERNEL_SKINNY, 2) == 0
    # From 65 to 256 tokens the skinny kernel for rows of at most 128 block
    # pairs and at most 128 row tiles (every token tile in workgroups of its
    # own, one split, no workspace); the GEMM otherwise.
    assert q8.q8_0_matmul_plan(4096, 2048, 65, 1 << 40) == (q8.KERNEL_SKINNY, 1)
    assert q8.q8_0_matmul_plan(8192, 4096, 256, 1 << 40) == (q8.KERNEL_SKINNY, 1)
    assert q8.q8_0_matmul_workspace_bytes(4096, 1024, 200) == 0
    assert q8.q8_0_matmul_plan(4096, 2048, 257, 1 << 40)[0] == q8.KERNEL_MFMA
    assert q8.q8_0_matmul_plan(8256, 2048, 128, 1 << 40)[0] == q8.KERNEL_MFMA
    assert q8.q8_0_matmul_plan(4096, 4128, 128, 1 << 40)[0] == q8.KERNEL_MFMA
    # Long rows with at most 32 row tiles: two splits up to 128 tokens.
    assert q8.q8_0_matmul_plan(32768, 1024, 128, 1 << 40) == (q8.KERNEL_SKINNY, 2)
    assert q8.q8_0_matmul_plan(32768, 1024, 128, 0) == (q8.KERNEL_SKINNY, 1)
    assert q8.q8_0_matmul_plan(32768, 1024, 129, 1 << 40)[0] == q8.KERNEL_MFMA
    assert q8.q8_0_matmul_plan(16384, 2048, 100, 1 << 40)[0] == q8.KERNEL_MFMA
    # A K split above 64 tokens: partials and a counter per (row tile, token
    # tile); at most 1024 counters.
    assert q8.q8_0_matmul_debug_workspace_bytes(4096, 2048, 100, q8.KERNEL_SKINNY, 2) == \
        4096 + 2 * 64 * 4 * 4096
    assert q8.q8_0_matmul_debug_workspace_bytes(4096, 4096, 256, q8.KERNEL_SKINNY, 2) == \
        4096 + 2 * 128 * 8 * 4096
    assert q8.q8_0_matmul_debug_workspace_bytes(4096, 4128, 256, q8.KERNEL_SKINNY, 2) == 0
    # Above that the tiled GEMM; split-K aims for 256 workgroups.
    assert q8.q8_0_matmul_plan(1024, 32768, 128, 1 << 40) == (q8.KERNEL_MFMA, 1)
    assert q8.q8_0_matmul_plan(4096, 2048, 4096, 1 << 40) == (q8.KERNEL_MFMA, 1)
    v, s = q8.q8_0_matmul_plan(32768, 1024, 2048, 1 << 40)
    assert v == q8.KERNEL_MFMA and s == 8
    need = q8.q8_0_matmul_workspace_bytes(32768, 1024, 2048)
    assert need == 4096 + 8 * 1024 * 2048 * 4
    # Without workspace the split falls back to 1; with some, to what fits.
    assert q8.q8_0_matmul_plan(32768, 1024, 2048, 0) == (q8.KERNEL_MFMA, 1)
    assert q8.q8_0_matmul_plan(32768, 1024, 2048, 4096 + 3 * 1024 * 2048 * 4) == (q8.KERNEL_MFMA, 3)
    assert q8.q8_0_matmul_debug_workspace_bytes(32768, 1024, 2048, q8.KERNEL_MFMA, 3) == \
        4096 + 3 * 1024 * 2048 * 4
    # Block counts that are not whole pairs take the generic kernel.
    assert q8.q8_0_matmul_plan(96, 64, 1, 0) == (q8.KERNEL_GENERIC, 1)
    assert q8.q8_0_matmul_plan(96, 64, 100, 0) == (q8.KERNEL_GENERIC, 1)
    assert q8.q8_0_matmul_workspace_bytes(1024, 32768, 1) == 0


def test_valid_call_without_device_reports_nodev(q8):
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a device is present")
    lib = q8.raw_library()
    assert lib.q8_0_matmul(FAKE, FAKE, 32, 4, FAKE, 1, None, 0, None) == q8.Q8_0_ENODEV
    assert lib.q8_0_quantize_act(FAKE, FAKE, 1, 32, None) == q8.Q8_0_ENODEV
    items = (q8.MatmulItem * 2)(q8.MatmulItem(FAKE, FAKE, FAKE, None, 1024, 256),
                                q8.MatmulItem(FAKE, FAKE, None, FAKE, 8192, 64))
    assert lib.q8_0_matmul_list(items, 2, 1, None) == q8.Q8_0_ENODEV
    assert lib.q8_0_debug_poison_lds(0xFFFFFFFF, None) == q8.Q8_0_ENODEV
    assert lib.q8_0_debug_read_lds(FAKE, 4, None) == q8.Q8_0_ENODEV


def test_oracle_is_not_imported_by_the_product():
    # The product path never loads the oracle.
    for root, _, files in os.walk(os.path.join(ROOT, "q8_quantized_matmul_amd")):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(root, f), encoding="utf-8").read()
                assert "oracle" not in text.replace("oracles", ""), f


def test_probe_validation(q8):
    lib = q8.raw_library()
    assert lib.q8_0_probe_read(None, 64, FAKE, None) == q8.Q8_0_EINVAL
    assert lib.q8_0_probe_read(FAKE, 0, FAKE, None) == q8.Q8_0_EINVAL
    assert lib.q8_0_probe_read(FAKE, 100, FAKE, None) == q8.Q8_0_EINVAL   # not a multiple of 16
    assert lib.q8_0_probe_read(FAKE + 4, 64, FAKE, None) == q8.Q8_0_EINVAL
    assert lib.q8_0_probe_read(FAKE, 64, None, None) == q8.Q8_0_EINVAL
    assert lib.q8_0_probe_mfma_i8(0, FAKE, None) == q8.Q8_0_EINVAL
    assert lib.q8_0_probe_mfma_i8(10, None, None) == q8.Q8_0_EINVAL
    assert lib.q8_0_probe_mfma_mix(0, 1, FAKE, None) == q8.Q8_0_EINVAL
    assert lib.q8_0_probe_mfma_mix(10, 3, FAKE, None) == q8.Q8_0_EINVAL
    assert lib.q8_0_probe_mfma_mix(10, 1, None, None) == q8.Q8_0_EINVAL
    assert lib.q8_0_probe_launch(0, FAKE, None) == q8.Q8_0_EINVAL
    assert lib.q8_0_probe_launch(65537, FAKE, None) == q8.Q8_0_EINVAL
    assert lib.q8_0_probe_launch(16, None, None) == q8.Q8_0_EINVAL
    assert lib.q8_0_debug_read_lds(None, 4, None) == q8.Q8_0_EINVAL
    assert lib.q8_0_debug_read_lds(FAKE + 2, 4, None) == q8.Q8_0_EINVAL
    assert lib.q8_0_debug_read_lds(FAKE, 0, None) == q8.Q8_0_EINVAL
    assert lib.q8_0_debug_read_lds(FAKE, 4097, None) == q8.Q8_0_EINVAL
