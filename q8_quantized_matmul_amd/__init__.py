"""Python binding of libq8_0.so, the gfx950 Q8_0 quantized matmul library.

Argument marshalling only: every function forwards torch tensors' device
pointers and the current torch stream to the C ABI in include/q8_0.h, where
all checks and all computation happen.  torch supplies device memory (outputs
and scratch are allocated with torch when the caller passes none) and
streams.  If the library has not been built, importing this package raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libq8_0.so")

BLOCK_ELEMS = 32
BLOCK_BYTES = 34

Q8_0_OK = 0
Q8_0_EINVAL = -1
Q8_0_EALIGN = -2
Q8_0_ELAUNCH = -3
Q8_0_EWORKSPACE = -4
Q8_0_ENODEV = -5

KERNEL_AUTO = 0
KERNEL_GENERIC = 1
KERNEL_MATVEC = 2
KERNEL_MFMA = 3
KERNEL_SKINNY = 4


class Q8Error(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: {q8_0_strerror(code)} (status {code})")
        self.code = code


if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing; build it with `python q8_quantized_matmul_amd/build.py`")

_lib = ctypes.CDLL(LIB_PATH)
_i64, _i32, _vp, _sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t

LIST_MAX = 16


class MoeFfnArgs(ctypes.Structure):
    """struct q8_0_moe_ffn_args."""
    _fields_ = [("out", _vp), ("gate_w", _vp), ("up_w", _vp), ("down_w", _vp),
                ("n_expert", _i32), ("n_used", _i32), ("d_model", _i64), ("d_ff", _i64),
                ("n_tok", _i64), ("selected", _vp), ("weights", _vp), ("x_q", _vp),
                ("clamp", ctypes.c_float), ("mid", _vp), ("mid_q", _vp), ("y", _vp)]


class MatmulItem(ctypes.Structure):
    """struct q8_0_matmul_item."""
    _fields_ = [("out", _vp), ("w", _vp), ("x", _vp), ("x_q", _vp), ("in_dim", _i64),
                ("out_dim", _i64)]

_sig = {
    "q8_0_quantize_act": ([_vp, _vp, _i64, _i64, _vp], ctypes.c_int),
    "q8_0_matmul_workspace_bytes": ([_i64, _i64, _i64], _sz),
    "q8_0_matmul": ([_vp, _vp, _i64, _i64, _vp, _i64, _vp, _sz, _vp], ctypes.c_int),
    "q8_0_moe_workspace_bytes": ([_i64, _i32, _i32], _sz),
    "q8_0_moe_grouped": ([_vp, _vp, _i32, _i64, _i64, _vp, _i32, _vp, _i32, _i64, _vp, _sz, _vp],
                         ctypes.c_int),
    "q8_0_moe_grouped_noalloc": ([_vp, _vp, _i32, _i64, _i64, _vp, _i32, _vp, _i32, _i64, _vp,
                                  _vp], ctypes.c_int),
    "q8_0_matmul_debug": ([_vp, _vp, _vp, _i64, _i64, _vp, _i64, _vp, _sz, _i32, _i32, _vp],
                          ctypes.c_int),
    "q8_0_moe_grouped_debug": ([_vp, _vp, _vp, _i32, _i64, _i64, _vp, _i32, _vp, _i32, _i64, _vp,
                                _sz, _vp], ctypes.c_int),
    "q8_0_matmul_debug_workspace_bytes": ([_i64, _i64, _i64, _i32, _i32], _sz),
    "q8_0_matmul_plan": ([_i64, _i64, _i64, _sz, ctypes.POINTER(_i32), ctypes.POINTER(_i32)],
                         ctypes.c_int),
    "q8_0_matmul_list": ([ctypes.POINTER(MatmulItem), _i32, _i64, _vp], ctypes.c_int),
    "q8_0_moe_ffn_workspace_bytes": ([_i64, _i32, _i32, _i64, _i64], _sz),
    "q8_0_moe_ffn": ([ctypes.POINTER(MoeFfnArgs), _vp, _sz, _vp], ctypes.c_int),
    "q8_0_probe_read": ([_vp, _sz, _vp, _vp], ctypes.c_int),
    "q8_0_probe_launch": ([_i32, _vp, _vp], ctypes.c_int),
    "q8_0_probe_mfma_i8": ([_i32, _vp, _vp], ctypes.c_int),
    "q8_0_probe_mfma_mix": ([_i32, _i32, _vp, _vp], ctypes.c_int),
    "q8_0_debug_poison_lds": ([ctypes.c_uint32, _vp], ctypes.c_int),
    "q8_0_debug_read_lds": ([_vp, _i32, _vp], ctypes.c_int),
    "q8_0_strerror": ([ctypes.c_int], ctypes.c_char_p),
}
for _name, (_args, _res) in _sig.items():
    _fn = getattr(_lib, _name)
    _fn.argtypes = _args
    _fn.restype = _res

EXPORTED = tuple(_sig)


def raw_library() -> ctypes.CDLL:
    return _lib


def q8_0_strerror(code: int) -> str:
    return _lib.q8_0_strerror(int(code)).decode()


def row_bytes(in_dim: int) -> int:
    return in_dim // BLOCK_ELEMS * BLOCK_BYTES


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _dev(t: torch.Tensor, name: str, dtype=None) -> int:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}")
    return t.data_ptr()


def _check(code: int, where: str) -> None:
    if code != Q8_0_OK:
        raise Q8Error(code, where)


def q8_0_quantize_act(x: torch.Tensor, out: torch.Tensor = None) -> torch.Tensor:
    """x: fp32 [n_tok][in_dim] -> uint8 [n_tok][in_dim/32*34] Q8_0 blocks."""
    if x.dim() == 1:
        x = x.unsqueeze(0)
    n_tok, in_dim = x.shape
    if out is None:
        out = torch.empty((n_tok, row_bytes(in_dim)), dtype=torch.uint8, device=x.device)
    _check(_lib.q8_0_quantize_act(_dev(out, "out"), _dev(x, "x", torch.float32), n_tok, in_dim,
                                  _stream()), "q8_0_quantize_act")
    return out


def q8_0_matmul_workspace_bytes(in_dim: int, out_dim: int, n_tok: int) -> int:
    return int(_lib.q8_0_matmul_workspace_bytes(in_dim, out_dim, n_tok))


def q8_0_matmul_debug_workspace_bytes(in_dim: int, out_dim: int, n_tok: int, variant: int = 0,
                                      split_k: int = 0) -> int:
    return int(_lib.q8_0_matmul_debug_workspace_bytes(in_dim, out_dim, n_tok, variant, split_k))


def matmul_workspace(in_dim: int, out_dim: int, n_tok: int, device="cuda", variant: int = 0,
                     split_k: int = 0) -> torch.Tensor:
    """A zero-filled workspace for this shape and plan (the split-K counters
    at its start must be zero before first use; calls leave them zero)."""
    n = q8_0_matmul_debug_workspace_bytes(in_dim, out_dim, n_tok, variant, split_k)
    return torch.zeros(max(n, 1), dtype=torch.uint8, device=device)


def _nbytes(t: torch.Tensor) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def q8_0_matmul(w: torch.Tensor, x_q: torch.Tensor, in_dim: int, out_dim: int, n_tok: int,
                out: torch.Tensor = None, workspace: torch.Tensor = None) -> torch.Tensor:
    """out fp32 [n_tok][out_dim] = Q8_0 weights [out_dim][in_dim] x Q8_0 x_q [n_tok][in_dim].
    Without a workspace, one is allocated (and zero-filled) only for plans that
    need it; plans that need none (the matvec) get a null pointer."""
    if out is None:
        out = torch.empty((n_tok, out_dim), dtype=torch.float32, device=w.device)
    if workspace is None and q8_0_matmul_workspace_bytes(in_dim, out_dim, n_tok) > 0:
        workspace = matmul_workspace(in_dim, out_dim, n_tok, w.device)
    _check(_lib.q8_0_matmul(_dev(out, "out", torch.float32), _dev(w, "w"), in_dim, out_dim,
                            _dev(x_q, "x_q"), n_tok, _dev(workspace, "workspace"),
                            _nbytes(workspace), _stream()),
           "q8_0_matmul")
    return out


def q8_0_matmul_debug(w, x_q, in_dim, out_dim, n_tok, variant=KERNEL_AUTO, split_k=0,
                      blocksums=True, out=None, workspace=None):
    """q8_0_matmul with a forced kernel variant / split; returns (out, blocksums or None)."""
    if out is None:
        out = torch.empty((n_tok, out_dim), dtype=torch.float32, device=w.device)
    bs = None
    if blocksums:
        bs = torch.empty((n_tok, out_dim, in_dim // BLOCK_ELEMS), dtype=torch.int32,
                         device=w.device)
    if workspace is None and q8_0_matmul_debug_workspace_bytes(in_dim, out_dim, n_tok, variant,
                                                               split_k) > 0:
        workspace = matmul_workspace(in_dim, out_dim, n_tok, w.device, variant, split_k)
    _check(_lib.q8_0_matmul_debug(_dev(out, "out", torch.float32),
                                  _dev(bs, "blocksums") if bs is not None else None,
                                  _dev(w, "w"), in_dim, out_dim, _dev(x_q, "x_q"), n_tok,
                                  _dev(workspace, "workspace"),
                                  _nbytes(workspace), variant, split_k,
                                  _stream()), "q8_0_matmul_debug")
    return out, bs


def q8_0_matmul_list(items, n_tok: int) -> None:
    """Several projections in as few launches as possible.  items: sequence of
    dicts with keys out (fp32 [n_tok][out_dim]), w, in_dim, out_dim and x (fp32
    [n_tok][in_dim]) and/or x_q (uint8 Q8_0 rows); missing keys mean NULL.
    Outputs (and x_q when x is given) are written in place."""
    arr = (MatmulItem * max(len(items), 1))()
    for i, it in enumerate(items):
        arr[i] = MatmulItem(_dev(it.get("out"), "out", torch.float32), _dev(it.get("w"), "w"),
                            _dev(it.get("x"), "x", torch.float32), _dev(it.get("x_q"), "x_q"),
                            int(it["in_dim"]), int(it["out_dim"]))
    _check(_lib.q8_0_matmul_list(arr, len(items), n_tok, _stream()), "q8_0_matmul_list")


def q8_0_matmul_plan(in_dim: int, out_dim: int, n_tok: int, workspace_bytes: int):
    v, s = _i32(0), _i32(0)
    _check(_lib.q8_0_matmul_plan(in_dim, out_dim, n_tok, workspace_bytes, ctypes.byref(v),
                                 ctypes.byref(s)), "q8_0_matmul_plan")
    return v.value, s.value


def q8_0_moe_workspace_bytes(n_tok: int, n_used: int, n_expert: int) -> int:
    return int(_lib.q8_0_moe_workspace_bytes(n_tok, n_used, n_expert))


def expert_table(mats) -> torch.Tensor:
    """Device int64 table of expert weight base pointers from a list of tensors
    (or from one stacked [n_expert, ...] tensor).  The table holds raw device
    addresses: the tensors must stay alive as long as the table is used."""
    if isinstance(mats, torch.Tensor):
        base = mats.data_ptr()
        stride = mats[0].numel() * mats.element_size()
        ptrs = [base + e * stride for e in range(mats.shape[0])]
        device = mats.device
    else:
        ptrs = [m.data_ptr() for m in mats]
        device = mats[0].device
    return torch.tensor(ptrs, dtype=torch.int64).to(device)


def _moe(debug, table, n_expert, selected, x_q, in_dim, out_dim, x_rows, out, workspace):
    n_tok, n_used = selected.shape
    if out is None:
        out = torch.empty((n_tok, n_used, out_dim), dtype=torch.float32, device=x_q.device)
    if workspace is None:
        workspace = torch.empty(q8_0_moe_workspace_bytes(n_tok, n_used, n_expert),
                                dtype=torch.uint8, device=x_q.device)
    args = [_dev(table, "expert table", torch.int64), n_expert, in_dim, out_dim,
            _dev(selected, "selected", torch.int32), n_used, _dev(x_q, "x_q"), x_rows, n_tok,
            _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
            _stream()]
    bs = None
    if debug:
        bs = torch.empty((n_tok * n_used, out_dim, in_dim // BLOCK_ELEMS), dtype=torch.int32,
                         device=x_q.device)
        _check(_lib.q8_0_moe_grouped_debug(_dev(out, "out", torch.float32), _dev(bs, "bs"),
                                           *args), "q8_0_moe_grouped_debug")
    else:
        _check(_lib.q8_0_moe_grouped(_dev(out, "out", torch.float32), *args), "q8_0_moe_grouped")
    return out, bs, workspace


def q8_0_moe_grouped(table, n_expert, selected, x_q, in_dim, out_dim, x_rows=0, out=None,
                     workspace=None):
    """out fp32 [n_tok][n_used][out_dim]; table = expert_table(...).  Returns
    (out, workspace); workspace[:4] viewed as int32 counts invalid expert ids."""
    out, _, ws = _moe(False, table, n_expert, selected, x_q, in_dim, out_dim, x_rows, out,
                      workspace)
    return out, ws


MOE_STATIC_SCRATCH_BYTES = 1 << 20


def q8_0_moe_grouped_noalloc(table, n_expert, selected, x_q, in_dim, out_dim, x_rows=0,
                             out=None, n_invalid=None):
    """q8_0_moe_grouped with the routing tables in the library's static
    device array (the C call allocates nothing).  out is allocated here when
    not given; n_invalid, an optional device int32 tensor of one element,
    receives the count of invalid expert ids.  Returns out."""
    n_tok, n_used = selected.shape
    if out is None:
        out = torch.empty((n_tok, n_used, out_dim), dtype=torch.float32, device=x_q.device)
    _check(_lib.q8_0_moe_grouped_noalloc(
        _dev(out, "out", torch.float32), _dev(table, "expert table", torch.int64), n_expert,
        in_dim, out_dim, _dev(selected, "selected", torch.int32), n_used, _dev(x_q, "x_q"),
        x_rows, n_tok, _dev(n_invalid, "n_invalid", torch.int32), _stream()),
        "q8_0_moe_grouped_noalloc")
    return out


def q8_0_moe_grouped_debug(table, n_expert, selected, x_q, in_dim, out_dim, x_rows=0, out=None,
                           workspace=None):
    return _moe(True, table, n_expert, selected, x_q, in_dim, out_dim, x_rows, out, workspace)


def moe_invalid_count(workspace: torch.Tensor) -> int:
    return int(workspace[:4].view(torch.int32).item())


def q8_0_moe_ffn_workspace_bytes(n_tok: int, n_used: int, n_expert: int, d_model: int,
                                 d_ff: int) -> int:
    return int(_lib.q8_0_moe_ffn_workspace_bytes(n_tok, n_used, n_expert, d_model, d_ff))


def q8_0_moe_ffn(gate_table, up_table, down_table, n_expert, selected, weights, x_q, d_model,
                 d_ff, clamp=0.0, out=None, mid=None, mid_q=None, y=None, workspace=None):
    """Routed expert FFN: out fp32 [n_tok][d_model].  Tables from expert_table();
    selected int32 / weights fp32 [n_tok][n_used]; mid, mid_q, y optional
    intermediate buffers.  Returns (out, workspace); workspace[:4] as int32
    counts invalid expert ids."""
    n_tok, n_used = selected.shape
    if out is None:
        out = torch.empty((n_tok, d_model), dtype=torch.float32, device=x_q.device)
    if workspace is None:
        workspace = torch.empty(
            max(q8_0_moe_ffn_workspace_bytes(n_tok, n_used, n_expert, d_model, d_ff), 256),
            dtype=torch.uint8, device=x_q.device)
    args = MoeFfnArgs(_dev(out, "out", torch.float32), _dev(gate_table, "gate table", torch.int64),
                      _dev(up_table, "up table", torch.int64),
                      _dev(down_table, "down table", torch.int64), n_expert, n_used, d_model,
                      d_ff, n_tok, _dev(selected, "selected", torch.int32),
                      _dev(weights, "weights", torch.float32), _dev(x_q, "x_q"), float(clamp),
                      _dev(mid, "mid", torch.float32), _dev(mid_q, "mid_q"),
                      _dev(y, "y", torch.float32))
    _check(_lib.q8_0_moe_ffn(ctypes.byref(args), _dev(workspace, "workspace"),
                             workspace.numel() * workspace.element_size(), _stream()),
           "q8_0_moe_ffn")
    return out, workspace


PROBE_MFMA_OPS_PER_ITER = 512 * 4 * 4 * 65536  # integer ops per round of q8_0_probe_mfma_i8


def q8_0_probe_read(buf: torch.Tensor, sink: torch.Tensor) -> None:
    """Streaming read of the whole (contiguous, 16-byte aligned) device tensor."""
    _check(_lib.q8_0_probe_read(_dev(buf, "buf"), buf.numel() * buf.element_size(),
                                _dev(sink, "sink"), _stream()), "q8_0_probe_read")


def q8_0_probe_launch(workgroups: int, sink: torch.Tensor) -> None:
    """An empty launch of `workgroups` workgroups: the fixed cost of a launch."""
    _check(_lib.q8_0_probe_launch(int(workgroups), _dev(sink, "sink"), _stream()),
           "q8_0_probe_launch")


def q8_0_probe_mfma_i8(iters: int, sink: torch.Tensor) -> None:
    _check(_lib.q8_0_probe_mfma_i8(int(iters), _dev(sink, "sink"), _stream()),
           "q8_0_probe_mfma_i8")


def q8_0_probe_mfma_mix(iters: int, mix: int, sink: torch.Tensor) -> None:
    """The GEMM's per-tile-block instruction mix (mix 1, or 2 with VALU
    conversion; 0 = int8 MFMA alone), int8 work per round as
    PROBE_MFMA_OPS_PER_ITER."""
    _check(_lib.q8_0_probe_mfma_mix(int(iters), int(mix), _dev(sink, "sink"), _stream()),
           "q8_0_probe_mfma_mix")


DEBUG_LDS_DWORDS = 8192  # Q8_0_DEBUG_LDS_DWORDS


def q8_0_debug_poison_lds(pattern: int) -> None:
    """Fill every compute unit's LDS with the 32-bit pattern (race tests)."""
    _check(_lib.q8_0_debug_poison_lds(int(pattern) & 0xFFFFFFFF, _stream()),
           "q8_0_debug_poison_lds")


def q8_0_debug_read_lds(seen: torch.Tensor, workgroups: int) -> None:
    """Copy the unwritten LDS of `workgroups` workgroups into seen (int32,
    workgroups * DEBUG_LDS_DWORDS elements)."""
    assert seen.numel() * seen.element_size() >= workgroups * DEBUG_LDS_DWORDS * 4
    _check(_lib.q8_0_debug_read_lds(_dev(seen, "seen"), int(workgroups), _stream()),
           "q8_0_debug_read_lds")
