"""ctypes binding of libfavor.so (include/favor.h).

Argument marshalling only: every arithmetic step runs in the library's
HIP kernels.  torch is used for device memory (tensors, workspace) and
for the current HIP stream.  There is no CPU fallback: if the library is
missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Tuple

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
# FAVOR_LIB may name another build of the same library (the host-sanitizer
# build that the ABI tests load in a child process)
LIB_PATH = os.environ.get("FAVOR_LIB") or os.path.join(PKG, "libfavor.so")

FAVOR_OK = 0
FAVOR_ERR_INVALID_ARG = -1
FAVOR_ERR_UNSUPPORTED = -2
FAVOR_ERR_WORKSPACE = -3
FAVOR_ERR_ALIAS = -4
FAVOR_ERR_HIP = -5

DTYPE = {"f32": 0, "bf16": 1}
KIND = {"trig": 0, "relu": 1, "positive": 2}
PATH = {"auto": 0, "generic": 1, "mfma": 2, "small": 3}
PATH_NAME = {v: k for k, v in PATH.items()}

EXPORTS = (
    "favor_version", "favor_status_string", "favor_orf_omega",
    "favor_attention_workspace_bytes", "favor_attention_workspace_bytes_ex",
    "favor_attention", "favor_attention_ex", "favor_attention_resolve_path",
    "favor_profile_attention", "favor_embed_bf16", "favor_linear_bf16",
    "favor_pack_weight_bf16", "favor_embed_linear_bf16",
    "favor_attention_train", "favor_attention_backward_saved",
    "favor_attention_backward_workspace_bytes", "favor_attention_backward",
    "favor_attention_backward_workspace_bytes_ex", "favor_attention_backward_ex",
    "favor_attention_noalloc",
)


class FavorError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


_lib: Optional[ctypes.CDLL] = None

_c_int, _c_size, _vp = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p


def _declare(lib: ctypes.CDLL) -> None:
    i, z, p = _c_int, _c_size, _vp
    sig = {
        "favor_version": (i, []),
        "favor_status_string": (ctypes.c_char_p, [i]),
        "favor_orf_omega": (i, [p, p, i, i, p]),
        "favor_attention_workspace_bytes": (z, [i] * 8),
        "favor_attention_workspace_bytes_ex": (z, [i] * 9),
        "favor_attention": (i, [p, p, p, p, p] + [i] * 8 + [p, z, p]),
        "favor_attention_ex": (i, [p, p, p, p, p] + [i] * 8 + [p, z, p, i]),
        "favor_attention_resolve_path": (i, [i] * 9),
        "favor_profile_attention": (i, [p, p, p, p, p] + [i] * 8 + [p, z, p, i, i, p, p, i, p]),
        "favor_embed_bf16": (i, [p, p, p, i, i, i, p]),
        "favor_linear_bf16": (i, [p, p, p, i, i, i, i, i, i, p]),
        "favor_pack_weight_bf16": (i, [p, p, i, i, p]),
        "favor_embed_linear_bf16": (i, [p, p, i, p, p, i, i, i, i, i, i, p]),
        "favor_attention_backward_workspace_bytes": (z, [i] * 8),
        "favor_attention_backward": (i, [p] * 8 + [i] * 8 + [p, z, p]),
        "favor_attention_backward_workspace_bytes_ex": (z, [i] * 9),
        "favor_attention_backward_ex": (i, [p] * 8 + [i] * 8 + [p, z, p, i]),
        "favor_attention_train": (i, [p] * 6 + [i] * 8 + [p, z, p, i]),
        "favor_attention_backward_saved": (i, [p] * 10 + [i] * 8 + [p, z, p, i]),
        "favor_attention_noalloc": (i, [p, p, p, p, p] + [i] * 8 + [p, i]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args


def lib() -> ctypes.CDLL:
    """Load libfavor.so (after torch, so both share torch's HIP runtime)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -m linear_kernelized_attention_amd.build`")
        import torch  # noqa: F401  -- load torch's HIP runtime first
        handle = ctypes.CDLL(LIB_PATH, mode=ctypes.RTLD_GLOBAL)
        _declare(handle)
        _lib = handle
    return _lib


def loaded_hip_runtimes() -> List[str]:
    """Paths of every libamdhip64 mapped in this process (should be one)."""
    paths = set()
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    paths.add(line.split()[-1])
    except OSError:
        pass
    return sorted(paths)


def status_string(status: int) -> str:
    return lib().favor_status_string(int(status)).decode()


def _check(status: int, what: str) -> None:
    if status != FAVOR_OK:
        raise FavorError(status, what)


# ----------------------------------------------------------------- host ORF
def favor_orf_omega(gaussian: np.ndarray, radii: np.ndarray, m: int) -> np.ndarray:
    """Omega [m, d] float32 from raw Gaussian blocks and chi(d) radii."""
    g = np.ascontiguousarray(gaussian, dtype=np.float64)
    r = np.ascontiguousarray(radii, dtype=np.float64)
    n_blocks, d, d2 = g.shape
    if d != d2 or n_blocks * d < m or r.size < m:
        raise ValueError("gaussian must be [ceil(m/d), d, d] and radii [m]")
    out = np.empty((m, d), dtype=np.float32)
    _check(lib().favor_orf_omega(g.ctypes.data, r.ctypes.data, int(m), int(d), out.ctypes.data),
           "favor_orf_omega")
    return out


# ----------------------------------------------------------------- attention
def _torch_dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return DTYPE["f32"]
    if t.dtype == torch.bfloat16:
        return DTYPE["bf16"]
    raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")


def _stream_ptr(device) -> int:
    import torch
    return torch.cuda.current_stream(device).cuda_stream


def _validate(q, k, v, omega):
    import torch
    for name, t in (("q", q), ("k", k), ("v", v), ("omega", omega)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be on the GPU")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must all be [B, H, L, d]")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    if omega.dtype != torch.float32 or omega.dim() != 2 or omega.shape[1] != q.shape[3]:
        raise ValueError("omega must be float32 [m, d]")
    if not (q.device == k.device == v.device == omega.device):
        raise ValueError("all tensors must be on one device")


def favor_attention_workspace_bytes(B, H, L, d, m, dtype="bf16", kind="trig", causal=False,
                                    path="auto") -> int:
    return int(lib().favor_attention_workspace_bytes_ex(
        B, H, L, d, m, DTYPE[dtype], KIND[kind], int(bool(causal)), PATH[path]))


def favor_attention_resolve_path(B, H, L, d, m, dtype="bf16", kind="trig", causal=False,
                                 path="auto") -> str:
    r = lib().favor_attention_resolve_path(B, H, L, d, m, DTYPE[dtype], KIND[kind],
                                           int(bool(causal)), PATH[path])
    _check(FAVOR_OK if r > 0 else r, "favor_attention_resolve_path")
    return PATH_NAME[r]


def _call_args(q, k, v, omega, kind, causal, path, out, workspace):
    import torch
    _validate(q, k, v, omega)
    B, H, L, d = q.shape
    m = omega.shape[0]
    dt = _torch_dtype_code(q)
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor like q")
    need = int(lib().favor_attention_workspace_bytes_ex(B, H, L, d, m, dt, KIND[kind],
                                                        int(bool(causal)), PATH[path]))
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    args = [q.data_ptr(), k.data_ptr(), v.data_ptr(), omega.data_ptr(), out.data_ptr(),
            B, H, L, d, m, dt, KIND[kind], int(bool(causal)),
            workspace.data_ptr(), workspace.numel(), _stream_ptr(q.device), PATH[path]]
    return args, out, workspace


def favor_attention(q, k, v, omega, kind: str = "trig", causal: bool = False, path: str = "auto",
                    out=None, workspace=None, den=None):
    """FAVOR attention of [B, H, L, d] float32/bf16 tensors on the GPU.

    With den (a float32 [B, H, L] tensor, or True to allocate one) the row
    normalisers D_ii are written too, and (out, den) is returned: the pair
    favor_attention_backward(..., saved=(out, den)) reuses."""
    import torch
    args, out, _ = _call_args(q, k, v, omega, kind, causal, path, out, workspace)
    if den is None or den is False:
        _check(lib().favor_attention_ex(*args), "favor_attention")
        return out
    if den is True:
        den = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    if den.dtype != torch.float32 or tuple(den.shape) != tuple(q.shape[:3]) or not den.is_contiguous():
        raise ValueError("den must be a contiguous float32 [B, H, L] tensor")
    _check(lib().favor_attention_train(*args[:5], den.data_ptr(), *args[5:]), "favor_attention_train")
    return out, den


def favor_attention_noalloc(q, k, v, omega, kind: str = "trig", causal: bool = False,
                            path: str = "auto", out=None):
    """favor_attention through the entry point that allocates nothing: the
    library's fixed per-device scratch replaces the workspace (calls that
    overlap in time on one device race; see include/favor.h)."""
    import torch
    _validate(q, k, v, omega)
    B, H, L, d = q.shape
    m = omega.shape[0]
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor like q")
    _check(lib().favor_attention_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), omega.data_ptr(),
                                         out.data_ptr(), B, H, L, d, m, _torch_dtype_code(q),
                                         KIND[kind], int(bool(causal)), _stream_ptr(q.device),
                                         PATH[path]), "favor_attention_noalloc")
    return out


def favor_attention_backward_workspace_bytes(B, H, L, d, m, dtype="bf16", kind="trig",
                                             causal=False, path="auto") -> int:
    return int(lib().favor_attention_backward_workspace_bytes_ex(
        B, H, L, d, m, DTYPE[dtype], KIND[kind], int(bool(causal)), PATH[path]))


def favor_attention_backward(q, k, v, omega, dout, kind: str = "trig", causal: bool = False,
                             path: str = "auto", workspace=None, grads=None, saved=None):
    """(dq, dk, dv) of sum(dout * favor_attention(q, k, v)) on the GPU; grads
    may supply the three output tensors; saved = (out, den) from
    favor_attention(..., den=True) skips recomputing the forward (MFMA)."""
    import torch
    _validate(q, k, v, omega)
    if dout.shape != q.shape or dout.dtype != q.dtype or not dout.is_contiguous():
        raise ValueError("dout must be a contiguous tensor like q")
    B, H, L, d = q.shape
    m = omega.shape[0]
    dt = _torch_dtype_code(q)
    if grads is None:
        grads = tuple(torch.empty_like(q) for _ in range(3))
    for t in grads:
        if t.shape != q.shape or t.dtype != q.dtype or not t.is_contiguous():
            raise ValueError("grads must be contiguous tensors like q")
    need = int(lib().favor_attention_backward_workspace_bytes_ex(B, H, L, d, m, dt, KIND[kind],
                                                                 int(bool(causal)), PATH[path]))
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    dq, dk, dv = grads
    tail = [dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, L, d, m, dt,
            KIND[kind], int(bool(causal)), workspace.data_ptr(), workspace.numel(),
            _stream_ptr(q.device), PATH[path]]
    head = [q.data_ptr(), k.data_ptr(), v.data_ptr(), omega.data_ptr()]
    if saved is None:
        _check(lib().favor_attention_backward_ex(*head, *tail), "favor_attention_backward")
    else:
        out, den = saved
        if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
            raise ValueError("saved out must be a contiguous tensor like q")
        if den.dtype != torch.float32 or tuple(den.shape) != tuple(q.shape[:3]) or not den.is_contiguous():
            raise ValueError("saved den must be a contiguous float32 [B, H, L] tensor")
        _check(lib().favor_attention_backward_saved(*head, out.data_ptr(), den.data_ptr(), *tail),
               "favor_attention_backward_saved")
    return dq, dk, dv


def favor_attention_backward_resolve_path(B, H, L, d, m, dtype="bf16", kind="trig",
                                          causal=False) -> str:
    """The kernel family favor_attention_backward runs ("mfma" or "generic")."""
    ws_m = favor_attention_backward_workspace_bytes(B, H, L, d, m, dtype, kind, causal, "mfma")
    return "mfma" if ws_m > 0 else "generic"


def favor_profile_attention(q, k, v, omega, kind="trig", causal=False, path="auto", iters=20,
                            out=None, workspace=None) -> List[Tuple[str, float]]:
    """[(kernel name, mean ms per launch)]: each kernel launched `iters`
    times back-to-back between two HIP events on the current stream."""
    args, out, _ = _call_args(q, k, v, omega, kind, causal, path, out, workspace)
    max_ph = 8
    ms = (ctypes.c_float * max_ph)()
    names = ctypes.create_string_buffer(48 * max_ph)
    n = ctypes.c_int(0)
    _check(lib().favor_profile_attention(*args, int(iters), ms, names, max_ph, ctypes.byref(n)),
           "favor_profile_attention")
    res = []
    for i in range(n.value):
        nm = names.raw[48 * i:48 * (i + 1)].split(b"\0", 1)[0].decode()
        res.append((nm, float(ms[i])))
    return res


# ------------------------------------------------------------ block helpers
def favor_embed_bf16(ids, table, out=None):
    import torch
    if ids.dtype != torch.int32 or table.dtype != torch.bfloat16:
        raise TypeError("ids must be int32 and table bfloat16")
    if not ids.is_contiguous() or not table.is_contiguous():
        raise ValueError("ids and table must be contiguous")
    n_tok = ids.numel()
    vocab, E = table.shape
    if out is None:
        out = torch.empty(*ids.shape, E, dtype=torch.bfloat16, device=table.device)
    _check(lib().favor_embed_bf16(ids.data_ptr(), table.data_ptr(), out.data_ptr(), n_tok, vocab, E,
                                  _stream_ptr(table.device)), "favor_embed_bf16")
    return out


def favor_pack_weight_bf16(w, out=None):
    """Wt = W^T for a bf16 [K, N] weight: the packed [N, K] layout of the
    projections (a device layout change)."""
    import torch
    if w.dtype != torch.bfloat16 or w.dim() != 2 or not w.is_contiguous():
        raise TypeError("w must be a contiguous 2-D bfloat16 tensor")
    K, N = w.shape
    if out is None:
        out = torch.empty(N, K, dtype=torch.bfloat16, device=w.device)
    elif out.numel() != K * N or not out.is_contiguous():
        raise ValueError("out must be contiguous with K*N elements")
    _check(lib().favor_pack_weight_bf16(w.data_ptr(), out.data_ptr(), K, N, _stream_ptr(w.device)),
           "favor_pack_weight_bf16")
    return out


def favor_linear_bf16(x, wt, M: int, N: int, K: int, in_heads: int = 0, out_heads: int = 0,
                      seq_len: int = 0, out=None):
    """Y = X Wt^T with a packed [N, K] weight and optional head-split layouts
    (see include/favor.h)."""
    import torch
    if x.dtype != torch.bfloat16 or wt.dtype != torch.bfloat16:
        raise TypeError("x and wt must be bfloat16")
    if not x.is_contiguous() or not wt.is_contiguous():
        raise ValueError("x and wt must be contiguous")
    if x.numel() != M * K or wt.numel() != K * N:
        raise ValueError("x must hold M*K and wt N*K elements")
    if out is None:
        out = torch.empty(M * N, dtype=torch.bfloat16, device=x.device)
    elif out.numel() != M * N:
        raise ValueError("out must hold M*N elements")
    _check(lib().favor_linear_bf16(x.data_ptr(), wt.data_ptr(), out.data_ptr(), M, N, K, in_heads,
                                   out_heads, seq_len, _stream_ptr(x.device)), "favor_linear_bf16")
    return out


def favor_embed_linear_bf16(ids, table, wt, out_heads: int = 0, head_dim: int = 0, seq_len: int = 0,
                            out=None):
    """Y = table[ids] Wt^T without storing table[ids]; head-split output in
    groups of out_heads * head_dim columns (see include/favor.h)."""
    import torch
    if ids.dtype != torch.int32 or table.dtype != torch.bfloat16 or wt.dtype != torch.bfloat16:
        raise TypeError("ids must be int32, table and wt bfloat16")
    if not (ids.is_contiguous() and table.is_contiguous() and wt.is_contiguous()):
        raise ValueError("ids, table and wt must be contiguous")
    M = ids.numel()
    vocab, K = table.shape
    N = wt.shape[0]
    if wt.numel() != N * K:
        raise ValueError("wt must be [N, K] with K the table width")
    if out is None:
        out = torch.empty(M * N, dtype=torch.bfloat16, device=table.device)
    elif out.numel() != M * N:
        raise ValueError("out must hold M*N elements")
    _check(lib().favor_embed_linear_bf16(ids.data_ptr(), table.data_ptr(), vocab, wt.data_ptr(),
                                         out.data_ptr(), M, N, K, out_heads, head_dim, seq_len,
                                         _stream_ptr(table.device)), "favor_embed_linear_bf16")
    return out


class BlockWeights:
    """Packed projection weights of a masked-LM block: wqkv_t [3E, E] (the
    Q, K and V weights' [out, in] rows stacked) and wo_t [E, E]."""

    def __init__(self, wqkv_t, wo_t):
        self.wqkv_t = wqkv_t
        self.wo_t = wo_t


def favor_block_weights(wq, wk, wv, wo) -> BlockWeights:
    """Pack the block's four [E, E] (x W convention) weights once."""
    import torch
    E = wq.shape[0]
    wqkv_t = torch.empty(3 * E, E, dtype=torch.bfloat16, device=wq.device)
    for i, w in enumerate((wq, wk, wv)):
        favor_pack_weight_bf16(w, out=wqkv_t[i * E:(i + 1) * E])
    return BlockWeights(wqkv_t, favor_pack_weight_bf16(wo))


def favor_performer_block(ids, embed, weights: BlockWeights, omega, heads: int, kind: str = "relu",
                          path: str = "auto"):
    """Masked-LM attention block: one fused gather + Q/K/V projection written
    head-split, FAVOR attention, output projection reading the head-split
    result."""
    B, L = ids.shape
    E = embed.shape[1]
    dh = E // heads
    M = B * L
    qkv = favor_embed_linear_bf16(ids, embed, weights.wqkv_t, heads, dh, L).view(3, B, heads, L, dh)
    o = favor_attention(qkv[0], qkv[1], qkv[2], omega, kind=kind, causal=False, path=path)
    y = favor_linear_bf16(o, weights.wo_t, M, E, E, heads, 0, L)
    return y.view(B, L, E)
