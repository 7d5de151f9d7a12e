"""Python binding of ``libspecfold.so`` (the folded multi-branch verification layer).

Argument marshalling only: every function checks tensor dtypes, devices and sizes, passes raw
device pointers and torch's current HIP stream to the C ABI declared in
``include/specfold.h``, and raises ``SpecfoldError`` on a non-zero status.  Every step of the
layer runs in the library's HIP kernels; there is no fallback of any kind -- importing this
module without the built library raises.

Shapes are passed as any object with the attributes n_branch, block, hidden, n_q_heads,
n_kv_heads, head_dim, ffn, prefix_len, rms_eps, rope_theta.
"""

from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libspecfold.so")

OK = 0
STATUS = {
    0: "OK", -1: "ERR_NULL", -2: "ERR_SHAPE", -3: "ERR_TREE", -4: "ERR_ALIGN",
    -5: "ERR_WORKSPACE", -6: "ERR_UNSUPPORTED", -7: "ERR_ALIAS", -8: "ERR_HIP",
}
MAX_BRANCHES = 64
MAX_BLOCK = 64

# every symbol include/specfold.h declares
EXPORTS = (
    "specfold_version", "specfold_status_str", "specfold_last_error", "specfold_workspace_bytes", "specfold_stage_count",
    "specfold_stage_name", "specfold_event_create", "specfold_event_destroy",
    "specfold_event_elapsed_ms", "specfold_gate", "specfold_compact", "specfold_compact_workspace_bytes",
    "specfold_resolve_sources",
    "specfold_sparse_qkv", "specfold_folded_attention", "specfold_out_proj", "specfold_sparse_ffn",
    "specfold_verify_layer", "specfold_verify_layer_noalloc", "specfold_embed", "specfold_head_workspace_bytes",
    "specfold_lm_head",
)
NOALLOC_SCRATCH_BYTES = 128 << 20


class SpecfoldError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib.specfold_status_str(status).decode() if _lib is not None else ""
        if status == -8 and _lib is not None:
            msg += "; " + _lib.specfold_last_error().decode()
        super().__init__(f"{where}: {STATUS.get(status, status)} ({msg})")


class Shape(ctypes.Structure):
    _fields_ = [("n_branch", ctypes.c_int32), ("block", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("ffn", ctypes.c_int32), ("prefix_len", ctypes.c_int32), ("rms_eps", ctypes.c_float),
                ("rope_theta", ctypes.c_float)]


class PrefixKV(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("k_stride_tok", ctypes.c_int64),
                ("k_stride_head", ctypes.c_int64), ("v_stride_tok", ctypes.c_int64),
                ("v_stride_head", ctypes.c_int64)]


class LayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("ln1", "w_qkv", "w_o", "ln2", "w_gate_up", "w_down")]


class LayerStats(ctypes.Structure):
    _fields_ = [("rho", ctypes.c_void_p), ("fold", ctypes.c_void_p), ("rec_count", ctypes.c_void_p),
                ("src_slot", ctypes.c_void_p)]


class Trace(ctypes.Structure):
    _fields_ = [("events", ctypes.POINTER(ctypes.c_void_p)), ("n_events", ctypes.c_int32)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run `python -m sparse_layer_rho_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, F32, SZ = ctypes.c_void_p, ctypes.c_float, ctypes.c_size_t
    pS = ctypes.POINTER(Shape)
    sig = {
        "specfold_version": ([], ctypes.c_int),
        "specfold_status_str": ([ctypes.c_int], ctypes.c_char_p),
        "specfold_last_error": ([], ctypes.c_char_p),
        "specfold_workspace_bytes": ([pS], SZ),
        "specfold_stage_count": ([], ctypes.c_int),
        "specfold_stage_name": ([ctypes.c_int], ctypes.c_char_p),
        "specfold_event_create": ([ctypes.POINTER(ctypes.c_void_p)], ctypes.c_int),
        "specfold_event_destroy": ([P], ctypes.c_int),
        "specfold_event_elapsed_ms": ([P, P, ctypes.POINTER(ctypes.c_float)], ctypes.c_int),
        "specfold_gate": ([pS, P, P, F32, P, P, P, P, P], ctypes.c_int),
        "specfold_compact": ([pS, P, P, P, P, P, P, SZ, P], ctypes.c_int),
        "specfold_compact_workspace_bytes": ([pS], SZ),
        "specfold_resolve_sources": ([pS, P, P, P, P, P, P], ctypes.c_int),
        "specfold_sparse_qkv": ([pS, P, P, P, P, P, P, P, P, P, P, SZ, P], ctypes.c_int),
        "specfold_folded_attention": ([pS, P, P, P, P, P, P, ctypes.POINTER(PrefixKV), P, P, P, SZ, P],
                                      ctypes.c_int),
        "specfold_out_proj": ([pS, P, P, P, P, P, SZ, P], ctypes.c_int),
        "specfold_sparse_ffn": ([pS, P, P, P, P, P, P, P, P, P, SZ, P], ctypes.c_int),
        "specfold_embed": ([pS, P, P, ctypes.c_int32, P, P], ctypes.c_int),
        "specfold_head_workspace_bytes": ([pS, ctypes.c_int32], SZ),
        "specfold_lm_head": ([pS, P, P, P, ctypes.c_int32, P, P, P, SZ, P], ctypes.c_int),
        "specfold_verify_layer": ([pS, P, ctypes.POINTER(LayerWeights), ctypes.POINTER(PrefixKV), P, F32, P,
                                   ctypes.POINTER(LayerStats), ctypes.POINTER(Trace), P, SZ, P], ctypes.c_int),
        "specfold_verify_layer_noalloc": ([pS, P, ctypes.POINTER(LayerWeights), ctypes.POINTER(PrefixKV), P, F32, P,
                                           ctypes.POINTER(LayerStats), ctypes.POINTER(Trace), P], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


_lib = _load()


def lib():
    return _lib


# ------------------------------------------------------------------ marshalling helpers

def make_shape(s) -> Shape:
    return Shape(int(s.n_branch), int(s.block), int(s.hidden), int(s.n_q_heads), int(s.n_kv_heads),
                 int(s.head_dim), int(s.ffn), int(s.prefix_len), float(s.rms_eps), float(s.rope_theta))


def _ptr(t, dtype=None, numel=None, name="tensor", optional=False):
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs {numel}")
    return t.data_ptr()


def _parent_host(parent, nb):
    p = torch.as_tensor(parent, dtype=torch.int32).cpu().contiguous()
    if p.numel() != nb:
        raise ValueError(f"parent map has {p.numel()} entries, shape says {nb} branches")
    return p


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(status, where):
    if status != OK:
        raise SpecfoldError(status, where)


def workspace_bytes(shape) -> int:
    sh = make_shape(shape)
    return int(_lib.specfold_workspace_bytes(ctypes.byref(sh)))


def new_workspace(shape, device="cuda") -> torch.Tensor:
    """Zero-filled workspace of the size every entry point of this shape needs."""
    n = workspace_bytes(shape)
    if n == 0:
        raise ValueError("shape not supported by the library")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def stage_names() -> list[str]:
    return [_lib.specfold_stage_name(i).decode() for i in range(_lib.specfold_stage_count())]


def prefix_view(k: torch.Tensor, v: torch.Tensor) -> PrefixKV:
    """Strided view of a prefix cache [P, Hkv, d] (any strides with a contiguous last dim)."""
    for name, t in (("prefix k", k), ("prefix v", v)):
        if t.dtype != torch.bfloat16 or not t.is_cuda or t.dim() != 3 or t.stride(2) != 1:
            raise ValueError(f"{name} must be a bf16 device tensor [P, Hkv, d] with unit last stride")
    return PrefixKV(k.data_ptr(), v.data_ptr(), k.stride(0), k.stride(1), v.stride(0), v.stride(1))


# ------------------------------------------------------------------ entry points

def gate(shape, parent, H, delta, rho, fold, inv_rms=None, rho_in=None):
    sh = make_shape(shape)
    R = shape.n_branch * shape.block
    par = _parent_host(parent, shape.n_branch)
    hp = _ptr(H, torch.bfloat16, R * shape.hidden, "H", optional=(rho_in is not None and inv_rms is None))
    st = _lib.specfold_gate(ctypes.byref(sh), ctypes.c_void_p(par.data_ptr()), hp, float(delta),
                            _ptr(rho_in, torch.float32, R, "rho_in", True), _ptr(rho, torch.float32, R, "rho"),
                            _ptr(fold, torch.uint8, R, "fold"), _ptr(inv_rms, torch.float32, R, "inv_rms", True),
                            _stream())
    _check(st, "specfold_gate")


def compact_workspace(shape, device="cuda"):
    """Scratch for ``compact`` (None when the shape needs none)."""
    n = int(_lib.specfold_compact_workspace_bytes(ctypes.byref(make_shape(shape))))
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def compact(shape, fold, rec_rows, rec_count, branch_off, row_slot, ws=None):
    """``ws``: a ``compact_workspace(shape)`` tensor; made here when not given (an allocation)."""
    sh = make_shape(shape)
    R = shape.n_branch * shape.block
    if ws is None:
        ws = compact_workspace(shape, fold.device)
    st = _lib.specfold_compact(ctypes.byref(sh), _ptr(fold, torch.uint8, R, "fold"),
                               _ptr(rec_rows, torch.int32, R, "rec_rows"), _ptr(rec_count, torch.int32, 1, "rec_count"),
                               _ptr(branch_off, torch.int32, shape.n_branch + 1, "branch_off"),
                               _ptr(row_slot, torch.int32, R, "row_slot"),
                               _ptr(ws, torch.uint8, None, "ws", True), 0 if ws is None else ws.numel(), _stream())
    _check(st, "specfold_compact")


def resolve_sources(shape, parent, fold, row_slot, src_branch, src_slot):
    sh = make_shape(shape)
    R = shape.n_branch * shape.block
    par = _parent_host(parent, shape.n_branch)
    st = _lib.specfold_resolve_sources(ctypes.byref(sh), ctypes.c_void_p(par.data_ptr()),
                                       _ptr(fold, torch.uint8, R, "fold"), _ptr(row_slot, torch.int32, R, "row_slot"),
                                       _ptr(src_branch, torch.int32, R, "src_branch"),
                                       _ptr(src_slot, torch.int32, R, "src_slot"), _stream())
    _check(st, "specfold_resolve_sources")


def sparse_qkv(shape, H, inv_rms, rec_rows, rec_count, ln1, w_qkv, q_c, k_c, v_c, ws):
    sh = make_shape(shape)
    R, D = shape.n_branch * shape.block, shape.hidden
    nq = (shape.n_q_heads + 2 * shape.n_kv_heads) * shape.head_dim
    st = _lib.specfold_sparse_qkv(
        ctypes.byref(sh), _ptr(H, torch.bfloat16, R * D, "H"), _ptr(inv_rms, torch.float32, R, "inv_rms"),
        _ptr(rec_rows, torch.int32, R, "rec_rows"), _ptr(rec_count, torch.int32, 1, "rec_count"),
        _ptr(ln1, torch.bfloat16, D, "ln1"), _ptr(w_qkv, torch.bfloat16, nq * D, "w_qkv"),
        _ptr(q_c, torch.bfloat16, R * shape.n_q_heads * shape.head_dim, "q_c"),
        _ptr(k_c, torch.bfloat16, R * shape.n_kv_heads * shape.head_dim, "k_c"),
        _ptr(v_c, torch.bfloat16, R * shape.n_kv_heads * shape.head_dim, "v_c"),
        _ptr(ws, torch.uint8, None, "ws"), ws.numel(), _stream())
    _check(st, "specfold_sparse_qkv")


def folded_attention(shape, q_c, k_c, v_c, rec_rows, rec_count, src_slot, prefix_k, prefix_v, attn, ws, lse=None):
    sh = make_shape(shape)
    R = shape.n_branch * shape.block
    pf = prefix_view(prefix_k, prefix_v) if shape.prefix_len > 0 else PrefixKV()
    st = _lib.specfold_folded_attention(
        ctypes.byref(sh), _ptr(q_c, torch.bfloat16, None, "q_c"), _ptr(k_c, torch.bfloat16, None, "k_c"),
        _ptr(v_c, torch.bfloat16, None, "v_c"), _ptr(rec_rows, torch.int32, R, "rec_rows"),
        _ptr(rec_count, torch.int32, 1, "rec_count"), _ptr(src_slot, torch.int32, R, "src_slot"), ctypes.byref(pf),
        _ptr(attn, torch.bfloat16, R * shape.n_q_heads * shape.head_dim, "attn"),
        _ptr(lse, torch.float32, R * shape.n_q_heads, "lse", True),
        _ptr(ws, torch.uint8, None, "ws"), ws.numel(), _stream())
    _check(st, "specfold_folded_attention")


def out_proj(shape, attn, H, w_o, h_mid, ws):
    sh = make_shape(shape)
    R, D = shape.n_branch * shape.block, shape.hidden
    st = _lib.specfold_out_proj(
        ctypes.byref(sh), _ptr(attn, torch.bfloat16, R * shape.n_q_heads * shape.head_dim, "attn"),
        _ptr(H, torch.bfloat16, R * D, "H"), _ptr(w_o, torch.bfloat16, D * shape.n_q_heads * shape.head_dim, "w_o"),
        _ptr(h_mid, torch.bfloat16, R * D, "h_mid"), _ptr(ws, torch.uint8, None, "ws"), ws.numel(), _stream())
    _check(st, "specfold_out_proj")


def sparse_ffn(shape, h_mid, rec_rows, rec_count, src_slot, ln2, w_gate_up, w_down, H_out, ws):
    sh = make_shape(shape)
    R, D, F = shape.n_branch * shape.block, shape.hidden, shape.ffn
    st = _lib.specfold_sparse_ffn(
        ctypes.byref(sh), _ptr(h_mid, torch.bfloat16, R * D, "h_mid"), _ptr(rec_rows, torch.int32, R, "rec_rows"),
        _ptr(rec_count, torch.int32, 1, "rec_count"), _ptr(src_slot, torch.int32, R, "src_slot"),
        _ptr(ln2, torch.bfloat16, D, "ln2"), _ptr(w_gate_up, torch.bfloat16, 2 * F * D, "w_gate_up"),
        _ptr(w_down, torch.bfloat16, D * F, "w_down"), _ptr(H_out, torch.bfloat16, R * D, "H_out"),
        _ptr(ws, torch.uint8, None, "ws"), ws.numel(), _stream())
    _check(st, "specfold_sparse_ffn")


def layer_weights_struct(w: dict) -> LayerWeights:
    return LayerWeights(*(_ptr(w[n], torch.bfloat16, None, n) for n in
                          ("ln1", "w_qkv", "w_o", "ln2", "w_gate_up", "w_down")))


def _layer_args(shape, parent, weights, prefix_k, prefix_v, stats):
    par = _parent_host(parent, shape.n_branch)
    lw = weights if isinstance(weights, LayerWeights) else layer_weights_struct(weights)
    pf = prefix_k if isinstance(prefix_k, PrefixKV) else (
        prefix_view(prefix_k, prefix_v) if shape.prefix_len > 0 else PrefixKV())
    R = shape.n_branch * shape.block
    st_obj = None
    if stats:
        st_obj = LayerStats(_ptr(stats.get("rho"), torch.float32, R, "rho", True),
                            _ptr(stats.get("fold"), torch.uint8, R, "fold", True),
                            _ptr(stats.get("rec_count"), torch.int32, 1, "rec_count", True),
                            _ptr(stats.get("src_slot"), torch.int32, R, "src_slot", True))
    return par, lw, pf, st_obj


def verify_layer_noalloc(shape, parent, weights, prefix_k, prefix_v, H_in, delta, H_out, stats=None, trace=None):
    """``verify_layer`` without a workspace: the library's own device scratch array serves as
    workspace (see ``specfold_verify_layer_noalloc``); calls on one device must not overlap."""
    sh = make_shape(shape)
    R, D = shape.n_branch * shape.block, shape.hidden
    par, lw, pf, st_obj = _layer_args(shape, parent, weights, prefix_k, prefix_v, stats)
    status = _lib.specfold_verify_layer_noalloc(
        ctypes.byref(sh), ctypes.c_void_p(par.data_ptr()), ctypes.byref(lw), ctypes.byref(pf),
        _ptr(H_in, torch.bfloat16, R * D, "H_in"), float(delta), _ptr(H_out, torch.bfloat16, R * D, "H_out"),
        ctypes.byref(st_obj) if st_obj is not None else None, ctypes.byref(trace) if trace is not None else None,
        _stream())
    _check(status, "specfold_verify_layer_noalloc")


def verify_layer(shape, parent, weights, prefix_k, prefix_v, H_in, delta, H_out, ws, stats=None, trace=None):
    """One folded verification layer.  ``weights`` is a dict of bf16 device tensors (or a
    prebuilt ``LayerWeights``); ``stats`` an optional dict with any of rho (f32 [R]), fold
    (u8 [R]), rec_count (i32 [1]), src_slot (i32 [R]); ``trace`` an optional ``Trace``."""
    sh = make_shape(shape)
    R, D = shape.n_branch * shape.block, shape.hidden
    par = _parent_host(parent, shape.n_branch)
    lw = weights if isinstance(weights, LayerWeights) else layer_weights_struct(weights)
    pf = prefix_k if isinstance(prefix_k, PrefixKV) else (
        prefix_view(prefix_k, prefix_v) if shape.prefix_len > 0 else PrefixKV())
    st_ptr = None
    if stats:
        st_obj = LayerStats(_ptr(stats.get("rho"), torch.float32, R, "rho", True),
                            _ptr(stats.get("fold"), torch.uint8, R, "fold", True),
                            _ptr(stats.get("rec_count"), torch.int32, 1, "rec_count", True),
                            _ptr(stats.get("src_slot"), torch.int32, R, "src_slot", True))
        st_ptr = ctypes.byref(st_obj)
    status = _lib.specfold_verify_layer(
        ctypes.byref(sh), ctypes.c_void_p(par.data_ptr()), ctypes.byref(lw), ctypes.byref(pf),
        _ptr(H_in, torch.bfloat16, R * D, "H_in"), float(delta), _ptr(H_out, torch.bfloat16, R * D, "H_out"),
        st_ptr, ctypes.byref(trace) if trace is not None else None,
        _ptr(ws, torch.uint8, None, "ws"), ws.numel(), _stream())
    _check(status, "specfold_verify_layer")


# ------------------------------------------------------------------ either side of the stack

def embed(shape, tokens, E, H):
    """H[r] = E[tokens[r]] (NaN rows for ids outside [0, V)); tokens int32 [R], E bf16 [V, D]."""
    sh = make_shape(shape)
    R, D = shape.n_branch * shape.block, shape.hidden
    V = E.shape[0]
    st = _lib.specfold_embed(ctypes.byref(sh), _ptr(tokens, torch.int32, R, "tokens"),
                             _ptr(E, torch.bfloat16, V * D, "E"), V, _ptr(H, torch.bfloat16, R * D, "H"), _stream())
    _check(st, "specfold_embed")


def head_workspace(shape, vocab, device="cuda") -> torch.Tensor:
    n = int(_lib.specfold_head_workspace_bytes(ctypes.byref(make_shape(shape)), int(vocab)))
    if n == 0:
        raise ValueError("shape or vocabulary not supported by the library")
    return torch.empty(n, dtype=torch.uint8, device=device)


def lm_head(shape, H, ln_f, w_lm, token, logit, ws):
    """Final RMSNorm, LM head and greedy token of every row: token int32 [R], logit f32 [R]."""
    sh = make_shape(shape)
    R, D = shape.n_branch * shape.block, shape.hidden
    V = w_lm.shape[0]
    st = _lib.specfold_lm_head(ctypes.byref(sh), _ptr(H, torch.bfloat16, R * D, "H"),
                               _ptr(ln_f, torch.bfloat16, D, "ln_f"), _ptr(w_lm, torch.bfloat16, V * D, "w_lm"), V,
                               _ptr(token, torch.int32, R, "token"), _ptr(logit, torch.float32, R, "logit"),
                               _ptr(ws, torch.uint8, None, "ws"), ws.numel(), _stream())
    _check(st, "specfold_lm_head")


# ------------------------------------------------------------------ per-launch timing

class StageTimer:
    """HIP events around every launch of ``verify_layer`` (pass ``.trace`` to it)."""

    def __init__(self):
        n = 2 * _lib.specfold_stage_count()
        self._ev = (ctypes.c_void_p * n)()
        for k in range(n):
            h = ctypes.c_void_p()
            _check(_lib.specfold_event_create(ctypes.byref(h)), "specfold_event_create")
            self._ev[k] = h
        self.trace = Trace(ctypes.cast(self._ev, ctypes.POINTER(ctypes.c_void_p)), n)
        self.names = stage_names()

    def elapsed_ms(self) -> dict:
        out = {}
        for k, name in enumerate(self.names):
            ms = ctypes.c_float()
            _check(_lib.specfold_event_elapsed_ms(self._ev[2 * k], self._ev[2 * k + 1], ctypes.byref(ms)),
                   "specfold_event_elapsed_ms")
            out[name] = ms.value
        return out

    def close(self):
        for k in range(len(self._ev)):
            if self._ev[k]:
                _lib.specfold_event_destroy(self._ev[k])
                self._ev[k] = None
