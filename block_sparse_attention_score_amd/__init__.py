"""Python binding of libspark_attn.so (two-branch block-sparse attention forward for MI355X).

Argument marshalling only: every step of the computation runs in the library's HIP kernels.
PyTorch provides device memory and the current stream.  The library must be built
(``python -m block_sparse_attention_score_amd.build``); loading fails loudly otherwise.

Low-level functions carry the C names (``spark_attn_pool`` ...) and take pre-allocated tensors.
The convenience functions ``pool``, ``select``, ``attend``, ``forward``, ``reblock`` and
``gather_rows`` allocate their outputs with torch and call the same entry points.
"""
from __future__ import annotations

import ctypes
import os

import torch  # loaded first so the library binds to the HIP runtime torch already uses

_PKG = os.path.dirname(os.path.abspath(__file__))
# SPARK_ATTN_LIB names another build of the library to load (the sanitizer test loads one whose
# host code is instrumented)
LIB_PATH = os.environ.get("SPARK_ATTN_LIB") or os.path.join(_PKG, "libspark_attn.so")

BF16, FP32 = 0, 1
POOL_MEAN, POOL_REWEIGHT = 0, 1


class SparkAttnParams(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int), ("H", ctypes.c_int), ("N", ctypes.c_int), ("d", ctypes.c_int),
        ("n_sink", ctypes.c_int), ("block", ctypes.c_int), ("topk_ratio", ctypes.c_float),
        ("pool_mode", ctypes.c_int), ("dtype", ctypes.c_int), ("scale", ctypes.c_float),
        ("block_k", ctypes.c_int),
    ]


class SparkAttnError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed: {status_str(status)} ({status})")


EXPORTS = (
    "spark_attn_num_blocks", "spark_attn_num_key_blocks", "spark_attn_topk_count", "spark_attn_workspace_size",
    "spark_attn_status_str", "spark_attn_pool", "spark_attn_select", "spark_attn_pack", "spark_attn_pool_pack",
    "spark_attn_attend", "spark_attn_forward", "spark_attn_forward_kv", "spark_attn_reblock",
    "spark_attn_gather_rows", "spark_attn_select_tau", "spark_attn_attend_var", "spark_attn_forward_tau",
    "spark_attn_fp8_scales", "spark_attn_pack_fp8", "spark_attn_attend_fp8", "spark_attn_forward_fp8",
    "spark_attn_pool_fp8_scales", "spark_attn_select_noalloc",
)

_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m block_sparse_attention_score_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(SparkAttnParams)
        vp, sz = ctypes.c_void_p, ctypes.c_size_t
        sig = {
            "spark_attn_num_blocks": ([P], ctypes.c_int),
            "spark_attn_num_key_blocks": ([P], ctypes.c_int),
            "spark_attn_topk_count": ([ctypes.c_int, ctypes.c_float], ctypes.c_int),
            "spark_attn_workspace_size": ([P, ctypes.c_int], sz),
            "spark_attn_status_str": ([ctypes.c_int], ctypes.c_char_p),
            "spark_attn_pool": ([P] + [vp] * 9 + [vp], ctypes.c_int),
            "spark_attn_select": ([P, vp, vp, vp, vp, vp, sz, vp], ctypes.c_int),
            "spark_attn_select_noalloc": ([P, vp, vp, vp, vp], ctypes.c_int),
            "spark_attn_pack": ([P, vp, vp, vp, vp, vp, vp, sz, vp], ctypes.c_int),
            "spark_attn_pool_pack": ([P] + [vp] * 10 + [sz, vp], ctypes.c_int),
            "spark_attn_attend": ([P, vp, vp, sz, vp, vp, vp, vp, vp], ctypes.c_int),
            "spark_attn_forward": ([P, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp], ctypes.c_int),
            "spark_attn_forward_kv": ([P, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp], ctypes.c_int),
            "spark_attn_reblock": ([P, vp, vp, vp, vp, sz, vp], ctypes.c_int),
            "spark_attn_gather_rows": ([P, vp, vp, vp, vp], ctypes.c_int),
            "spark_attn_select_tau": ([P, ctypes.c_float, vp, vp, vp, vp, vp, vp, sz, vp], ctypes.c_int),
            "spark_attn_attend_var": ([P, vp, vp, sz, vp, vp, vp, vp, vp, vp], ctypes.c_int),
            "spark_attn_forward_tau": ([P, ctypes.c_float, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
                                       ctypes.c_int),
            "spark_attn_fp8_scales": ([P, vp, vp, vp, vp, vp], ctypes.c_int),
            "spark_attn_pool_fp8_scales": ([P] + [vp] * 10 + [vp], ctypes.c_int),
            "spark_attn_pack_fp8": ([P, vp, vp, vp, vp, vp, vp, vp, sz, vp], ctypes.c_int),
            "spark_attn_attend_fp8": ([P, vp, vp, sz, vp, vp, vp, vp, vp, vp], ctypes.c_int),
            "spark_attn_forward_fp8": ([P, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp], ctypes.c_int),
        }
        for name, (args, res) in sig.items():
            fn = getattr(L, name)
            fn.argtypes, fn.restype = args, res
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().spark_attn_status_str(status).decode()


def params(Q: torch.Tensor, n_sink: int, block: int, topk_ratio: float = 0.1,
           pool_mode: int = POOL_REWEIGHT, scale: float = 0.0, block_k: int = 0) -> SparkAttnParams:
    """block: query block size; block_k: key block size (0: the same as block)."""
    B, H, N, d = Q.shape
    if Q.dtype == torch.bfloat16:
        dt = BF16
    elif Q.dtype == torch.float32:
        dt = FP32
    else:
        raise TypeError(f"unsupported dtype {Q.dtype}")
    return SparkAttnParams(B, H, N, d, n_sink, block, float(topk_ratio), int(pool_mode), dt,
                           float(scale), int(block_k))


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("tensors must be contiguous device tensors")
    return ctypes.c_void_p(t.data_ptr())


_DTYPES = {BF16: torch.bfloat16, FP32: torch.float32}

# Buffer roles of the entry points: element count per (batch, head) from the block geometry, and
# element type (None: the parameters' dtype).  Layouts are those the C header documents.
_ROLES = {
    "tok": (lambda g: g["N"] * g["d"], None),          # Q, K, V, O, X, Y [B,H,N,d]
    "qblk": (lambda g: g["M"] * g["d"], torch.float32),   # q_mean [B,H,M,d]
    "kblk": (lambda g: g["Mk"] * g["d"], torch.float32),  # k_mean, k_sum, v_sum [B,H,M_k,d]
    "kbias": (lambda g: g["Mk"], torch.float32),          # bias [B,H,M_k]
    "head": (lambda g: g["d"], torch.float32),            # anchor [B,H,d]
    "route": (lambda g: g["M"] * g["K"], torch.int32),    # idx [B,H,M,K]
    "route_all": (lambda g: g["M"] * g["Mk"], torch.int32),  # variable route idx [B,H,M,M_k]
    "scores": (lambda g: g["M"] * g["Mk"], torch.float32),   # S [B,H,M,M_k]
    "rows": (lambda g: g["N"], torch.float32),            # lse [B,H,N]
    "perm": (lambda g: g["Nv"], torch.int32),             # perm [B,H,N_v]
    "counts": (lambda g: g["M"], torch.int32),            # counts [B,H,M]
    # the same, as inputs whose contents the kernels follow
    "route_in": (lambda g: g["M"] * g["K"], torch.int32),
    "route_all_in": (lambda g: g["M"] * g["Mk"], torch.int32),
    "perm_in": (lambda g: g["Nv"], torch.int32),
    "counts_in": (lambda g: g["M"], torch.int32),
    "stats": (lambda g: 2, torch.float32),                # (mu, sigma) [B,H,2]
    "amax": (lambda g: 3, torch.float32),                 # amax [B,H,3]
}


# SPARK_ATTN_CHECK=1: also check the contents of the index inputs the kernels follow (routes,
# counts, permutations) before every launch.  This costs a device-to-host synchronisation per
# call, so it is off by default.  The kernels themselves clamp route entries and counts to the
# key blocks and skip output rows with a permutation entry out of range, so bad indices give
# wrong values rather than memory faults; the check turns them into an error.
CHECK_CONTENTS = os.environ.get("SPARK_ATTN_CHECK", "0") == "1"


def check_contents(p, idx=None, counts=None, perm=None):
    """Raises ValueError unless the index inputs are what the C header documents: a route
    idx [B,H,M,K] of strictly ascending key blocks in [0, M_k) (with counts [B,H,M] in [0, M_k]:
    a variable route, whose row I holds counts[I] such entries), and a permutation perm [B,H,N_v]
    of row indices in [0, N_v).  Works on tensors of any device."""
    L = lib()
    M, Mk = L.spark_attn_num_blocks(ctypes.byref(p)), L.spark_attn_num_key_blocks(ctypes.byref(p))
    Nv = p.N - p.n_sink
    if perm is not None:
        pv = perm.reshape(p.B * p.H, -1)[:, :Nv]
        if pv.numel() and (int(pv.min()) < 0 or int(pv.max()) >= Nv):
            raise ValueError(f"perm: entries outside [0, {Nv})")
    if counts is not None:
        c = counts.reshape(-1)[:p.B * p.H * M]
        if c.numel() and (int(c.min()) < 0 or int(c.max()) > Mk):
            raise ValueError(f"counts: entries outside [0, {Mk}]")
    if idx is not None:
        width = Mk if counts is not None else L.spark_attn_topk_count(Mk, p.topk_ratio)
        rows = idx.reshape(p.B * p.H * M, -1)[:, :width].long()
        valid = torch.ones_like(rows, dtype=torch.bool)
        if counts is not None:
            valid = torch.arange(width, device=rows.device)[None, :] < counts.reshape(-1)[:rows.shape[0], None].long()
        if bool(((rows < 0) | (rows >= Mk))[valid].any()):
            raise ValueError(f"idx: route entries outside [0, {Mk})")
        if width > 1 and bool(((rows[:, 1:] <= rows[:, :-1]) & valid[:, 1:]).any()):
            raise ValueError("idx: route rows not strictly ascending")


def _validate(p, *args):
    """Checks (name, tensor, role) triples against the parameters before a launch: a tensor that
    is too small or of the wrong element type would otherwise be read or written out of bounds
    by the kernels, which receive bare pointers.  Invalid parameters are left to the library,
    which reports them with its own status."""
    L = lib()
    M, Mk = L.spark_attn_num_blocks(ctypes.byref(p)), L.spark_attn_num_key_blocks(ctypes.byref(p))
    if M < 1 or Mk < 1 or p.dtype not in _DTYPES:
        return
    g = dict(N=p.N, d=p.d, M=M, Mk=Mk, K=L.spark_attn_topk_count(Mk, p.topk_ratio), Nv=p.N - p.n_sink)
    for name, t, role in args:
        if t is None:
            continue
        per_head, dtype = _ROLES[role]
        dtype = dtype or _DTYPES[p.dtype]
        need = p.B * p.H * per_head(g)
        if t.dtype != dtype:
            raise TypeError(f"{name}: element type {t.dtype}, expected {dtype}")
        if t.numel() < need:
            raise ValueError(f"{name}: {t.numel()} elements, expected {need}")
    if CHECK_CONTENTS:  # index inputs the kernels follow (roles ending in _in)
        d = {role: t for _, t, role in args if t is not None and role != "perm_in"}
        check_contents(p, idx=d.get("route_in", d.get("route_all_in")), counts=d.get("counts_in"))
        for _, t, role in args:
            if t is not None and role == "perm_in":
                check_contents(p, perm=t)


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _check(name, status):
    if status != 0:
        raise SparkAttnError(name, status)


def num_blocks(p: SparkAttnParams) -> int:
    m = lib().spark_attn_num_blocks(ctypes.byref(p))
    _check("spark_attn_num_blocks", min(m, 0))
    return m


def num_key_blocks(p: SparkAttnParams) -> int:
    m = lib().spark_attn_num_key_blocks(ctypes.byref(p))
    _check("spark_attn_num_key_blocks", min(m, 0))
    return m


def topk_count(M: int, ratio: float) -> int:
    k = lib().spark_attn_topk_count(M, ratio)
    _check("spark_attn_topk_count", min(k, 0))
    return k


def workspace_size(p: SparkAttnParams, what: int) -> int:
    return lib().spark_attn_workspace_size(ctypes.byref(p), what)


# ---- C-named entry points (pre-allocated tensors) -------------------------------------------

def spark_attn_pool(p, Q, K, V, q_mean, k_mean, k_sum, v_sum, bias, anchor, stream=None):
    _validate(p, ("Q", Q, "tok"), ("K", K, "tok"), ("V", V, "tok"), ("q_mean", q_mean, "qblk"),
              ("k_mean", k_mean, "kblk"), ("k_sum", k_sum, "kblk"), ("v_sum", v_sum, "kblk"),
              ("bias", bias, "kbias"), ("anchor", anchor, "head"))
    _check("spark_attn_pool", lib().spark_attn_pool(
        ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(V), _ptr(q_mean), _ptr(k_mean), _ptr(k_sum),
        _ptr(v_sum), _ptr(bias), _ptr(anchor), _stream(stream)))


def spark_attn_select(p, q_mean, k_mean, idx, scores=None, workspace=None, stream=None):
    _validate(p, ("q_mean", q_mean, "qblk"), ("k_mean", k_mean, "kblk"), ("idx", idx, "route"),
              ("scores", scores, "scores"))
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("spark_attn_select", lib().spark_attn_select(
        ctypes.byref(p), _ptr(q_mean), _ptr(k_mean), _ptr(idx), _ptr(scores), _ptr(workspace),
        ws_bytes, _stream(stream)))


def spark_attn_select_noalloc(p, q_mean, k_mean, idx, stream=None):
    """spark_attn_select with the score matrix in the library's static scratch (no workspace)."""
    _validate(p, ("q_mean", q_mean, "qblk"), ("k_mean", k_mean, "kblk"), ("idx", idx, "route"))
    _check("spark_attn_select_noalloc", lib().spark_attn_select_noalloc(
        ctypes.byref(p), _ptr(q_mean), _ptr(k_mean), _ptr(idx), _stream(stream)))


def _nbytes(t):
    return t.numel() * t.element_size() if t is not None else 0


def spark_attn_pack(p, K, V, k_sum, v_sum, bias, packed, stream=None):
    _validate(p, ("K", K, "tok"), ("V", V, "tok"), ("k_sum", k_sum, "kblk"), ("v_sum", v_sum, "kblk"),
              ("bias", bias, "kbias"))
    _check("spark_attn_pack", lib().spark_attn_pack(
        ctypes.byref(p), _ptr(K), _ptr(V), _ptr(k_sum), _ptr(v_sum), _ptr(bias), _ptr(packed),
        _nbytes(packed), _stream(stream)))


def spark_attn_pool_pack(p, Q, K, V, q_mean, k_mean, k_sum, v_sum, bias, anchor, packed, stream=None):
    _validate(p, ("Q", Q, "tok"), ("K", K, "tok"), ("V", V, "tok"), ("q_mean", q_mean, "qblk"),
              ("k_mean", k_mean, "kblk"), ("k_sum", k_sum, "kblk"), ("v_sum", v_sum, "kblk"),
              ("bias", bias, "kbias"), ("anchor", anchor, "head"))
    _check("spark_attn_pool_pack", lib().spark_attn_pool_pack(
        ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(V), _ptr(q_mean), _ptr(k_mean), _ptr(k_sum),
        _ptr(v_sum), _ptr(bias), _ptr(anchor), _ptr(packed), _nbytes(packed), _stream(stream)))


def spark_attn_attend(p, Q, packed, idx, perm, O, lse=None, stream=None):
    _validate(p, ("Q", Q, "tok"), ("idx", idx, "route_in"), ("perm", perm, "perm_in"), ("O", O, "tok"),
              ("lse", lse, "rows"))
    _check("spark_attn_attend", lib().spark_attn_attend(
        ctypes.byref(p), _ptr(Q), _ptr(packed), _nbytes(packed), _ptr(idx), _ptr(perm), _ptr(O),
        _ptr(lse), _stream(stream)))


def spark_attn_forward(p, Q, K, V, perm, O, lse, idx_out, workspace, stream=None):
    _validate(p, ("Q", Q, "tok"), ("K", K, "tok"), ("V", V, "tok"), ("perm", perm, "perm_in"), ("O", O, "tok"),
              ("lse", lse, "rows"), ("idx_out", idx_out, "route"))
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("spark_attn_forward", lib().spark_attn_forward(
        ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(V), _ptr(perm), _ptr(O), _ptr(lse),
        _ptr(idx_out), _ptr(workspace), ws_bytes, _stream(stream)))


def spark_attn_forward_kv(p, Q, K, V, perm_q, perm_k, O, lse, idx_out, workspace, stream=None):
    _validate(p, ("Q", Q, "tok"), ("K", K, "tok"), ("V", V, "tok"), ("perm_q", perm_q, "perm_in"),
              ("perm_k", perm_k, "perm_in"), ("O", O, "tok"), ("lse", lse, "rows"), ("idx_out", idx_out, "route"))
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("spark_attn_forward_kv", lib().spark_attn_forward_kv(
        ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(V), _ptr(perm_q), _ptr(perm_k), _ptr(O), _ptr(lse),
        _ptr(idx_out), _ptr(workspace), ws_bytes, _stream(stream)))


def spark_attn_select_tau(p, tau, q_mean, k_mean, idx, counts, stats, workspace, stream=None):
    _validate(p, ("q_mean", q_mean, "qblk"), ("k_mean", k_mean, "kblk"), ("idx", idx, "route_all"),
              ("counts", counts, "counts"), ("stats", stats, "stats"))
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("spark_attn_select_tau", lib().spark_attn_select_tau(
        ctypes.byref(p), float(tau), _ptr(q_mean), _ptr(k_mean), _ptr(idx), _ptr(counts), _ptr(stats),
        _ptr(workspace), ws_bytes, _stream(stream)))


def spark_attn_attend_var(p, Q, packed, idx, counts, perm, O, lse, stream=None):
    _validate(p, ("Q", Q, "tok"), ("idx", idx, "route_all_in"), ("counts", counts, "counts_in"),
              ("perm", perm, "perm_in"), ("O", O, "tok"), ("lse", lse, "rows"))
    _check("spark_attn_attend_var", lib().spark_attn_attend_var(
        ctypes.byref(p), _ptr(Q), _ptr(packed), _nbytes(packed), _ptr(idx), _ptr(counts), _ptr(perm),
        _ptr(O), _ptr(lse), _stream(stream)))


def spark_attn_forward_tau(p, tau, Q, K, V, O, lse, idx_out, counts_out, workspace, stream=None):
    _validate(p, ("Q", Q, "tok"), ("K", K, "tok"), ("V", V, "tok"), ("O", O, "tok"), ("lse", lse, "rows"),
              ("idx_out", idx_out, "route_all"), ("counts_out", counts_out, "counts"))
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("spark_attn_forward_tau", lib().spark_attn_forward_tau(
        ctypes.byref(p), float(tau), _ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(lse), _ptr(idx_out),
        _ptr(counts_out), _ptr(workspace), ws_bytes, _stream(stream)))


def spark_attn_fp8_scales(p, Q, K, V, amax, stream=None):
    _validate(p, ("Q", Q, "tok"), ("K", K, "tok"), ("V", V, "tok"), ("amax", amax, "amax"))
    _check("spark_attn_fp8_scales", lib().spark_attn_fp8_scales(
        ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(V), _ptr(amax), _stream(stream)))


def spark_attn_pool_fp8_scales(p, Q, K, V, q_mean, k_mean, k_sum, v_sum, bias, anchor, amax, stream=None):
    _validate(p, ("Q", Q, "tok"), ("K", K, "tok"), ("V", V, "tok"), ("q_mean", q_mean, "qblk"),
              ("k_mean", k_mean, "kblk"), ("k_sum", k_sum, "kblk"), ("v_sum", v_sum, "kblk"),
              ("bias", bias, "kbias"), ("anchor", anchor, "head"), ("amax", amax, "amax"))
    _check("spark_attn_pool_fp8_scales", lib().spark_attn_pool_fp8_scales(
        ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(V), _ptr(q_mean), _ptr(k_mean), _ptr(k_sum),
        _ptr(v_sum), _ptr(bias), _ptr(anchor), _ptr(amax), _stream(stream)))


def spark_attn_pack_fp8(p, K, V, k_sum, v_sum, bias, amax, packed, stream=None):
    _validate(p, ("K", K, "tok"), ("V", V, "tok"), ("k_sum", k_sum, "kblk"), ("v_sum", v_sum, "kblk"),
              ("bias", bias, "kbias"), ("amax", amax, "amax"))
    _check("spark_attn_pack_fp8", lib().spark_attn_pack_fp8(
        ctypes.byref(p), _ptr(K), _ptr(V), _ptr(k_sum), _ptr(v_sum), _ptr(bias), _ptr(amax),
        _ptr(packed), _nbytes(packed), _stream(stream)))


def spark_attn_attend_fp8(p, Q, packed, idx, perm, amax, O, lse=None, stream=None):
    _validate(p, ("Q", Q, "tok"), ("idx", idx, "route_in"), ("perm", perm, "perm_in"), ("amax", amax, "amax"),
              ("O", O, "tok"), ("lse", lse, "rows"))
    _check("spark_attn_attend_fp8", lib().spark_attn_attend_fp8(
        ctypes.byref(p), _ptr(Q), _ptr(packed), _nbytes(packed), _ptr(idx), _ptr(perm), _ptr(amax),
        _ptr(O), _ptr(lse), _stream(stream)))


def spark_attn_forward_fp8(p, Q, K, V, perm, O, lse, idx_out, amax_out, workspace, stream=None):
    _validate(p, ("Q", Q, "tok"), ("K", K, "tok"), ("V", V, "tok"), ("perm", perm, "perm_in"), ("O", O, "tok"),
              ("lse", lse, "rows"), ("idx_out", idx_out, "route"), ("amax_out", amax_out, "amax"))
    _check("spark_attn_forward_fp8", lib().spark_attn_forward_fp8(
        ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(V), _ptr(perm), _ptr(O), _ptr(lse), _ptr(idx_out),
        _ptr(amax_out), _ptr(workspace), _nbytes(workspace), _stream(stream)))


def spark_attn_reblock(p, Q, K, perm, workspace, stream=None):
    _validate(p, ("Q", Q, "tok"), ("K", K, "tok"), ("perm", perm, "perm"))
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("spark_attn_reblock", lib().spark_attn_reblock(
        ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(perm), _ptr(workspace), ws_bytes,
        _stream(stream)))


def spark_attn_gather_rows(p, X, perm, Y, stream=None):
    _validate(p, ("X", X, "tok"), ("perm", perm, "perm_in"), ("Y", Y, "tok"))
    _check("spark_attn_gather_rows", lib().spark_attn_gather_rows(
        ctypes.byref(p), _ptr(X), _ptr(perm), _ptr(Y), _stream(stream)))


# ---- convenience wrappers (allocate outputs with torch) -------------------------------------

def pool(Q, K, V, n_sink, block, pool_mode=POOL_REWEIGHT, scale=0.0, stream=None, block_k=0):
    """q_mean [B,H,M,d]; k_mean, k_sum, v_sum [B,H,M_k,d], bias [B,H,M_k]; anchor [B,H,d]."""
    p = params(Q, n_sink, block, 1.0, pool_mode, scale, block_k)
    M, Mk = num_blocks(p), num_key_blocks(p)
    B, H, _, d = Q.shape
    f = dict(device=Q.device, dtype=torch.float32)
    out = {"q_mean": torch.empty(B, H, M, d, **f)}
    out.update({k: torch.empty(B, H, Mk, d, **f) for k in ("k_mean", "k_sum", "v_sum")})
    out["bias"] = torch.empty(B, H, Mk, **f)
    out["anchor"] = torch.empty(B, H, d, **f)
    spark_attn_pool(p, Q, K, V, out["q_mean"], out["k_mean"], out["k_sum"], out["v_sum"],
                    out["bias"], out["anchor"], stream)
    return out


def pool_pack(Q, K, V, n_sink, block, pool_mode=POOL_REWEIGHT, scale=0.0, stream=None, block_k=0):
    """pool() and pack() in one pass over K and V: (pooled dict as pool() returns, packed)."""
    p = params(Q, n_sink, block, 1.0, pool_mode, scale, block_k)
    M, Mk = num_blocks(p), num_key_blocks(p)
    B, H, _, d = Q.shape
    f = dict(device=Q.device, dtype=torch.float32)
    out = {"q_mean": torch.empty(B, H, M, d, **f)}
    out.update({k: torch.empty(B, H, Mk, d, **f) for k in ("k_mean", "k_sum", "v_sum")})
    out["bias"] = torch.empty(B, H, Mk, **f)
    out["anchor"] = torch.empty(B, H, d, **f)
    packed = torch.empty(workspace_size(p, 4), device=Q.device, dtype=torch.uint8)
    spark_attn_pool_pack(p, Q, K, V, out["q_mean"], out["k_mean"], out["k_sum"], out["v_sum"],
                         out["bias"], out["anchor"], packed, stream)
    return out, packed


def select(q_mean, k_mean, Q, n_sink, block, topk_ratio, with_scores=False, scale=0.0,
           stream=None, block_k=0):
    p = params(Q, n_sink, block, topk_ratio, POOL_REWEIGHT, scale, block_k)
    M, Mk = num_blocks(p), num_key_blocks(p)
    K = topk_count(Mk, topk_ratio)
    B, H = q_mean.shape[:2]
    idx = torch.empty(B, H, M, K, device=q_mean.device, dtype=torch.int32)
    if with_scores:
        S = torch.empty(B, H, M, Mk, device=q_mean.device, dtype=torch.float32)
        spark_attn_select(p, q_mean, k_mean, idx, S, None, stream)
        return idx, S
    ws = torch.empty(workspace_size(p, 3), device=q_mean.device, dtype=torch.uint8)
    spark_attn_select(p, q_mean, k_mean, idx, None, ws, stream)
    return idx


def pack(K, V, pooled, n_sink, block, scale=0.0, stream=None, block_k=0):
    p = params(K, n_sink, block, 1.0, POOL_REWEIGHT, scale, block_k)
    packed = torch.empty(workspace_size(p, 4), device=K.device, dtype=torch.uint8)
    spark_attn_pack(p, K, V, pooled["k_sum"], pooled["v_sum"], pooled["bias"], packed, stream)
    return packed


def attend(Q, K, V, pooled, idx, n_sink, block, topk_ratio, perm=None, scale=0.0, out=None,
           lse=None, stream=None, block_k=0):
    p = params(Q, n_sink, block, topk_ratio, POOL_REWEIGHT, scale, block_k)
    packed = pack(K, V, pooled, n_sink, block, scale, stream, block_k)
    O = out if out is not None else torch.empty_like(Q)
    spark_attn_attend(p, Q, packed, idx, perm, O, lse, stream)
    return O


def forward(Q, K, V, n_sink, block, topk_ratio, pool_mode=POOL_REWEIGHT, perm=None, scale=0.0,
            return_lse=False, return_idx=False, workspace=None, stream=None, perm_k=None, block_k=0):
    """Returns O (and lse [B,H,N] fp32, idx [B,H,M,K] int32 when asked).  perm: the partition of
    the queries (and of keys and values unless perm_k is given); perm_k: a separate key
    partition (spark_attn_forward_kv); block_k: key block size (0: block)."""
    p = params(Q, n_sink, block, topk_ratio, pool_mode, scale, block_k)
    M = num_blocks(p)
    Kk = topk_count(num_key_blocks(p), topk_ratio)
    B, H, N, _ = Q.shape
    O = torch.empty_like(Q)
    lse = torch.empty(B, H, N, device=Q.device, dtype=torch.float32) if return_lse else None
    idx = torch.empty(B, H, M, Kk, device=Q.device, dtype=torch.int32) if return_idx else None
    if workspace is None:
        permuted = perm is not None or perm_k is not None
        workspace = torch.empty(workspace_size(p, 2 if permuted else 0), device=Q.device,
                                dtype=torch.uint8)
    if perm_k is None:
        spark_attn_forward(p, Q, K, V, perm, O, lse, idx, workspace, stream)
    else:
        spark_attn_forward_kv(p, Q, K, V, perm, perm_k, O, lse, idx, workspace, stream)
    res = (O,)
    if return_lse:
        res += (lse,)
    if return_idx:
        res += (idx,)
    return res[0] if len(res) == 1 else res


def select_tau(q_mean, k_mean, Q, n_sink, block, tau, scale=0.0, with_stats=False, stream=None):
    """Adaptive-tau routes: (idx [B,H,M,M], counts [B,H,M]) (and stats [B,H,2] when asked)."""
    p = params(Q, n_sink, block, 1.0, POOL_REWEIGHT, scale)
    M = num_blocks(p)
    B, H = q_mean.shape[:2]
    idx = torch.full((B, H, M, M), -1, device=q_mean.device, dtype=torch.int32)
    counts = torch.empty(B, H, M, device=q_mean.device, dtype=torch.int32)
    stats = torch.empty(B, H, 2, device=q_mean.device, dtype=torch.float32)
    ws = torch.empty(workspace_size(p, 5), device=q_mean.device, dtype=torch.uint8)
    spark_attn_select_tau(p, tau, q_mean, k_mean, idx, counts, stats, ws, stream)
    return (idx, counts, stats) if with_stats else (idx, counts)


def forward_tau(Q, K, V, n_sink, block, tau, pool_mode=POOL_REWEIGHT, scale=0.0, return_lse=False,
                return_route=False, workspace=None, stream=None):
    """Forward with adaptive-tau routes.  Returns O (and lse, and (idx, counts) when asked)."""
    p = params(Q, n_sink, block, 1.0, pool_mode, scale)
    M = num_blocks(p)
    B, H, N, _ = Q.shape
    O = torch.empty_like(Q)
    lse = torch.empty(B, H, N, device=Q.device, dtype=torch.float32) if return_lse else None
    idx = counts = None
    if return_route:
        idx = torch.full((B, H, M, M), -1, device=Q.device, dtype=torch.int32)
        counts = torch.empty(B, H, M, device=Q.device, dtype=torch.int32)
    if workspace is None:
        workspace = torch.empty(workspace_size(p, 6), device=Q.device, dtype=torch.uint8)
    spark_attn_forward_tau(p, tau, Q, K, V, O, lse, idx, counts, workspace, stream)
    res = (O,)
    if return_lse:
        res += (lse,)
    if return_route:
        res += (idx, counts)
    return res[0] if len(res) == 1 else res


def fp8_scales(Q, K, V, n_sink, block, stream=None):
    """amax [B,H,3] (Q, K, V) of the per-head E4M3 carriers."""
    p = params(Q, n_sink, block)
    B, H = Q.shape[:2]
    amax = torch.empty(B, H, 3, device=Q.device, dtype=torch.float32)
    spark_attn_fp8_scales(p, Q, K, V, amax, stream)
    return amax


def pack_fp8(K, V, pooled, amax, n_sink, block, scale=0.0, stream=None, block_k=0):
    p = params(K, n_sink, block, 1.0, POOL_REWEIGHT, scale, block_k)
    packed = torch.empty(workspace_size(p, 9), device=K.device, dtype=torch.uint8)
    spark_attn_pack_fp8(p, K, V, pooled["k_sum"], pooled["v_sum"], pooled["bias"], amax, packed, stream)
    return packed


def forward_fp8(Q, K, V, n_sink, block, topk_ratio, pool_mode=POOL_REWEIGHT, perm=None, scale=0.0,
                return_lse=False, return_idx=False, return_amax=False, workspace=None, stream=None,
                block_k=0):
    """Forward with the exact branch, sinks and pseudo-keys on per-head E4M3 carriers.  Returns O
    (and lse, idx [B,H,M,K], amax [B,H,3] when asked)."""
    p = params(Q, n_sink, block, topk_ratio, pool_mode, scale, block_k)
    M = num_blocks(p)
    Kk = topk_count(num_key_blocks(p), topk_ratio)
    B, H, N, _ = Q.shape
    O = torch.empty_like(Q)
    lse = torch.empty(B, H, N, device=Q.device, dtype=torch.float32) if return_lse else None
    idx = torch.empty(B, H, M, Kk, device=Q.device, dtype=torch.int32) if return_idx else None
    amax = torch.empty(B, H, 3, device=Q.device, dtype=torch.float32) if return_amax else None
    if workspace is None:
        workspace = torch.empty(workspace_size(p, 8 if perm is not None else 7), device=Q.device,
                                dtype=torch.uint8)
    spark_attn_forward_fp8(p, Q, K, V, perm, O, lse, idx, amax, workspace, stream)
    res = (O,)
    if return_lse:
        res += (lse,)
    if return_idx:
        res += (idx,)
    if return_amax:
        res += (amax,)
    return res[0] if len(res) == 1 else res


def reblock(Q, K, n_sink, block, workspace=None, stream=None):
    p = params(Q, n_sink, block)
    B, H, N, _ = Q.shape
    perm = torch.empty(B, H, N - n_sink, device=Q.device, dtype=torch.int32)
    if workspace is None:
        workspace = torch.empty(max(workspace_size(p, 1), 256), device=Q.device, dtype=torch.uint8)
    spark_attn_reblock(p, Q, K, perm, workspace, stream)
    return perm


def gather_rows(X, perm, n_sink, block=128, stream=None):
    p = params(X, n_sink, block)
    Y = torch.empty_like(X)
    spark_attn_gather_rows(p, X, perm, Y, stream)
    return Y
