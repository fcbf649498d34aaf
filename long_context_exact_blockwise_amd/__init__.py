"""MI355X (gfx950) exact blockwise causal attention with ring-order merging and masked
sequence packing.

Thin ctypes binding over the C-ABI library `liblwm_attn.so` (include/lwm_attn.h).  The
functions named `lwm_attn_*` mirror the C entry points one to one and only marshal
arguments: torch tensors supply device memory and the current HIP stream, every
computation runs in the library's HIP kernels.  There is no CPU fallback: if the library
is missing or no GPU is present the calls raise.

Convenience layers on top of those calls:
  attention_forward / attention_backward -- table + forward (+ backward) for one sequence
  ring_share_forward                      -- one device's share of the LWM ring: a query
                                             chunk merged against KV chunks in ring order
  attention_decode                        -- few query rows against a long KV cache
  rope                                    -- RoPE rotation of Q or K by global position
                                             (also the rope_theta option of the forward and
                                             backward layers)
  packed_loss                             -- cross-entropy reweighted per packed sample,
                                             with its gradient
"""
from __future__ import annotations

import contextlib
import ctypes
import math
import os
from typing import List, Optional, Sequence, Tuple

_PKG = os.path.dirname(os.path.abspath(__file__))
# LWM_ATTN_LIBRARY names another build of the same library (the host-sanitizer build of the
# boundary tests); by default the in-tree build is loaded
LIB_PATH = os.environ.get("LWM_ATTN_LIBRARY") or os.path.join(_PKG, "liblwm_attn.so")
# the race-canary build of the bf16 kernels and the build with device checks (see build.py)
CANARY_LIB_PATH = os.path.join(_PKG, "liblwm_attn_canary.so")
DEBUG_LIB_PATH = os.path.join(_PKG, "liblwm_attn_debug.so")

LWM_BF16, LWM_F32 = 0, 1
LWM_OUT_FINAL, LWM_OUT_PARTIAL = 0, 1
LWM_TILE_SKIP, LWM_TILE_PARTIAL, LWM_TILE_FULL = 0, 1, 2
TABLE_BLOCK = 64

STATUS = {
    0: "LWM_OK", -1: "LWM_ERR_INVALID_ARG", -2: "LWM_ERR_SHAPE", -3: "LWM_ERR_ALIGNMENT",
    -4: "LWM_ERR_UNSUPPORTED", -5: "LWM_ERR_WORKSPACE", -6: "LWM_ERR_HIP",
}

EXPORTED = (
    "lwm_attn_block_table_bytes", "lwm_attn_build_block_table", "lwm_attn_fwd",
    "lwm_attn_merge_chunk", "lwm_attn_bwd_workspace_bytes", "lwm_attn_bwd",
    "lwm_attn_bwd_phase", "lwm_attn_status_string", "lwm_attn_version",
    "lwm_attn_decode_workspace_bytes", "lwm_attn_decode", "lwm_attn_rope",
    "lwm_attn_packed_loss_workspace_bytes", "lwm_attn_packed_loss", "lwm_attn_decode_noalloc",
    "lwm_attn_fwd_rope", "lwm_attn_bwd_rope", "lwm_attn_debug_status",
)
LWM_DEBUG_SELF_TEST = 1
DECODE_SCRATCH_BYTES = 64 << 20  # LWM_DECODE_SCRATCH_BYTES
LWM_BWD_DELTA, LWM_BWD_DQ, LWM_BWD_DKV = 0, 1, 2


class LwmError(RuntimeError):
    def __init__(self, call: str, status: int, message: str):
        super().__init__(f"{call} failed with {status}: {message}")
        self.status = status


class Desc(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("Sq", ctypes.c_int32),
        ("Sk", ctypes.c_int32), ("D", ctypes.c_int32),
        ("q_offset", ctypes.c_int64), ("k_offset", ctypes.c_int64),
        ("scale", ctypes.c_float), ("causal", ctypes.c_int32),
        ("block_q", ctypes.c_int32), ("block_k", ctypes.c_int32), ("dtype", ctypes.c_int32),
    ]


_lib = None
_opened = {}


def load_library(path: str = LIB_PATH):
    """Load the shared library (once) and declare its signatures; every wrapper below calls
    the library loaded first (or the one active_library() selects)."""
    global _lib
    if _lib is not None:
        return _lib
    _lib = _open_library(path)
    return _lib


@contextlib.contextmanager
def active_library(path: str):
    """Run the wrappers against another build of the library (the race-canary build or the
    build with device checks) inside a `with` block."""
    global _lib
    prev = _lib
    _lib = _open_library(path)
    try:
        yield _lib
    finally:
        _lib = prev


def _open_library(path: str):
    if path in _opened:
        return _opened[path]
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run `python -m long_context_exact_blockwise_amd.build`")
    lib = ctypes.CDLL(path)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    DP = ctypes.POINTER(Desc)
    sig = {
        "lwm_attn_block_table_bytes": (SZ, [DP]),
        "lwm_attn_build_block_table": (ctypes.c_int, [DP, P, P, P, P]),
        "lwm_attn_fwd": (ctypes.c_int, [DP, I32, P, P, P, P, P, P, P, P, P, P, P, P]),
        "lwm_attn_merge_chunk": (ctypes.c_int, [I64, I32, P, P, P, P, P, P, I32, I32, P, P, P]),
        "lwm_attn_bwd_workspace_bytes": (SZ, [DP]),
        "lwm_attn_bwd": (ctypes.c_int, [DP, P, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P]),
        "lwm_attn_bwd_phase": (ctypes.c_int, [DP, I32, P, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P]),
        "lwm_attn_decode_workspace_bytes": (SZ, [DP]),
        "lwm_attn_decode": (ctypes.c_int, [DP, P, P, P, P, P, P, P, P, P, SZ, P]),
        "lwm_attn_decode_noalloc": (ctypes.c_int, [DP, P, P, P, P, P, P, P, P, P]),
        "lwm_attn_fwd_rope": (ctypes.c_int, [DP, I32, ctypes.c_double, P, P, P, P, P, P, P, P, P, P,
                                             P, P]),
        "lwm_attn_bwd_rope": (ctypes.c_int, [DP, ctypes.c_double, P, P, P, P, P, P, P, P, P, P, P,
                                             P, P, P, P, SZ, P]),
        "lwm_attn_rope": (ctypes.c_int, [I32, I32, I32, I32, I32, I64, ctypes.c_double, I32, P, P, P]),
        "lwm_attn_packed_loss_workspace_bytes": (SZ, [I32, I32, I32, I32]),
        "lwm_attn_packed_loss": (ctypes.c_int, [I32, I32, I32, I32, I32, P, P, P, ctypes.c_float, P, P,
                                                P, P, SZ, P]),
        "lwm_attn_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "lwm_attn_version": (ctypes.c_int, []),
        "lwm_attn_debug_status": (ctypes.c_int, [ctypes.POINTER(ctypes.c_uint32), I32]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _opened[path] = lib
    return lib


def lwm_attn_debug_status(self_test: bool = False) -> Tuple[int, int, int]:
    """(status, words[0], words[1]) of the library's device-check records, read and cleared
    (lwm_attn_debug_status); status is LWM_ERR_UNSUPPORTED (-4) for a build without checks."""
    w = (ctypes.c_uint32 * 2)()
    rc = load_library().lwm_attn_debug_status(w, LWM_DEBUG_SELF_TEST if self_test else 0)
    return rc, int(w[0]), int(w[1])


def _check(call: str, rc: int):
    if rc != 0:
        msg = load_library().lwm_attn_status_string(rc).decode()
        raise LwmError(call, rc, msg)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("lwm_attn: tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("lwm_attn: tensors must be contiguous")
    return t.data_ptr()


def _stream(stream=None) -> Optional[int]:
    import torch

    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _dtype_code(dtype) -> int:
    import torch

    if dtype == torch.bfloat16:
        return LWM_BF16
    if dtype == torch.float32:
        return LWM_F32
    raise ValueError(f"unsupported dtype {dtype}")


def _torch_dtype(code: int):
    import torch

    return {LWM_BF16: torch.bfloat16, LWM_F32: torch.float32}.get(int(code))


def _expect(t, numel: int, dtype, name: str):
    """Raise ValueError unless t (when given) holds exactly `numel` elements of `dtype`: the
    C entry points take raw pointers and cannot see a buffer's size."""
    if t is None:
        return
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"lwm_attn: {name} has dtype {t.dtype}, expected {dtype}")
    if t.numel() != numel:
        raise ValueError(f"lwm_attn: {name} has {t.numel()} elements, expected {numel}")


def _expect_attention(desc: "Desc", q=None, k=None, v=None, seg_q=None, seg_k=None, table=None,
                      qlike=(), klike=(), rowf=(), accs=()):
    """Sizes and dtypes of attention buffers against desc: Q-shaped [B,H,Sq,D] and K-shaped
    [B,H,Sk,D] in the desc dtype, float32 per-row [B,H,Sq] and accumulators [B,H,Sq,D],
    int32 segment ids [B,Sq] / [B,Sk], and a table of at least the size query's bytes."""
    import torch

    dt = _torch_dtype(desc.dtype)
    nq = desc.B * desc.H * desc.Sq * desc.D
    nk = desc.B * desc.H * desc.Sk * desc.D
    _expect(q, nq, dt, "q")
    _expect(k, nk, dt, "k")
    _expect(v, nk, dt, "v")
    for name, t in qlike:
        _expect(t, nq, dt, name)
    for name, t in klike:
        _expect(t, nk, dt, name)
    for name, t in rowf:
        _expect(t, desc.B * desc.H * desc.Sq, torch.float32, name)
    for name, t in accs:
        _expect(t, nq, torch.float32, name)
    _expect(seg_q, desc.B * desc.Sq, torch.int32, "seg_q")
    _expect(seg_k, desc.B * desc.Sk, torch.int32, "seg_k")
    if table is not None and table.numel() * table.element_size() < lwm_attn_block_table_bytes(desc):
        raise ValueError("lwm_attn: table buffer smaller than lwm_attn_block_table_bytes(desc)")


def make_desc(B, H, Sq, Sk, D, dtype, *, scale=None, causal=True, q_offset=0, k_offset=0,
              block_q=TABLE_BLOCK, block_k=TABLE_BLOCK) -> Desc:
    return Desc(B, H, Sq, Sk, D, int(q_offset), int(k_offset),
                float(1.0 / math.sqrt(D) if scale is None else scale), int(bool(causal)),
                int(block_q), int(block_k), _dtype_code(dtype) if not isinstance(dtype, int) else dtype)


# ---------------------------------------------------------------------------------------
# one-to-one wrappers of the C entry points
# ---------------------------------------------------------------------------------------

def lwm_attn_block_table_bytes(desc: Desc) -> int:
    return int(load_library().lwm_attn_block_table_bytes(ctypes.byref(desc)))


def lwm_attn_build_block_table(desc: Desc, seg_q, seg_k, table=None, stream=None):
    """Builds the block table into `table` (uint8 device tensor; allocated when None)."""
    import torch

    n = lwm_attn_block_table_bytes(desc)
    if table is None:
        table = torch.empty(max(n, 16), dtype=torch.uint8, device=seg_q.device)
    elif table.numel() * table.element_size() < n:
        raise ValueError("table buffer too small")
    rc = load_library().lwm_attn_build_block_table(ctypes.byref(desc), _ptr(seg_q), _ptr(seg_k),
                                                   _ptr(table), _stream(stream))
    _check("lwm_attn_build_block_table", rc)
    return table


def lwm_attn_fwd(desc: Desc, mode: int, q, k, v, seg_q, seg_k, table, o=None, lse=None, m=None,
                 l=None, acc=None, stream=None):
    _expect_attention(desc, q, k, v, seg_q, seg_k, table, qlike=(("o", o),),
                      rowf=(("lse", lse), ("m", m), ("l", l)), accs=(("acc", acc),))
    rc = load_library().lwm_attn_fwd(ctypes.byref(desc), int(mode), _ptr(q), _ptr(k), _ptr(v),
                                     _ptr(seg_q), _ptr(seg_k), _ptr(table), _ptr(o), _ptr(lse),
                                     _ptr(m), _ptr(l), _ptr(acc), _stream(stream))
    _check("lwm_attn_fwd", rc)


def lwm_attn_fwd_rope(desc: Desc, mode: int, theta: float, q, k_rot, v, seg_q, seg_k, table, o=None,
                      lse=None, m=None, l=None, acc=None, stream=None):
    """lwm_attn_fwd with q unrotated (turned by RoPE at load) and k_rot turned already."""
    _expect_attention(desc, q, k_rot, v, seg_q, seg_k, table, qlike=(("o", o),),
                      rowf=(("lse", lse), ("m", m), ("l", l)), accs=(("acc", acc),))
    rc = load_library().lwm_attn_fwd_rope(ctypes.byref(desc), int(mode), float(theta), _ptr(q),
                                          _ptr(k_rot), _ptr(v), _ptr(seg_q), _ptr(seg_k),
                                          _ptr(table), _ptr(o), _ptr(lse), _ptr(m), _ptr(l),
                                          _ptr(acc), _stream(stream))
    _check("lwm_attn_fwd_rope", rc)


def lwm_attn_merge_chunk(rows: int, D: int, m, l, acc, mc=None, lc=None, accc=None,
                         finalize: bool = False, out_dtype: int = LWM_BF16, o=None, lse=None,
                         stream=None):
    rc = load_library().lwm_attn_merge_chunk(int(rows), int(D), _ptr(m), _ptr(l), _ptr(acc),
                                             _ptr(mc), _ptr(lc), _ptr(accc), int(bool(finalize)),
                                             int(out_dtype), _ptr(o), _ptr(lse), _stream(stream))
    _check("lwm_attn_merge_chunk", rc)


def lwm_attn_decode_workspace_bytes(desc: Desc) -> int:
    return int(load_library().lwm_attn_decode_workspace_bytes(ctypes.byref(desc)))


def lwm_attn_decode(desc: Desc, q, k, v, seg_q, seg_k, table, o, lse, workspace, stream=None):
    _expect_attention(desc, q, k, v, seg_q, seg_k, table, qlike=(("o", o),), rowf=(("lse", lse),))
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = load_library().lwm_attn_decode(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v),
                                        _ptr(seg_q), _ptr(seg_k), _ptr(table), _ptr(o), _ptr(lse),
                                        _ptr(workspace), ws_bytes, _stream(stream))
    _check("lwm_attn_decode", rc)


def lwm_attn_decode_noalloc(desc: Desc, q, k, v, seg_q, seg_k, table, o, lse, stream=None):
    """lwm_attn_decode with the slice states in the library's static device buffer: the call
    allocates nothing.  Calls that overlap on one GPU race on that buffer."""
    _expect_attention(desc, q, k, v, seg_q, seg_k, table, qlike=(("o", o),), rowf=(("lse", lse),))
    rc = load_library().lwm_attn_decode_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v),
                                                _ptr(seg_q), _ptr(seg_k), _ptr(table), _ptr(o),
                                                _ptr(lse), _stream(stream))
    _check("lwm_attn_decode_noalloc", rc)


def lwm_attn_rope(x, out, pos_offset: int, theta: float, inverse: bool = False, stream=None):
    """RoPE of x [B,H,S,D] (bf16 or float32) into out (may be x itself), row s at position
    pos_offset + s."""
    if x.dim() != 4 or out.shape != x.shape or out.dtype != x.dtype:
        raise ValueError("lwm_attn_rope: x and out must be [B,H,S,D] of one shape and dtype")
    B, H, S, D = x.shape
    rc = load_library().lwm_attn_rope(B, H, S, D, _dtype_code(x.dtype), int(pos_offset), float(theta),
                                      int(bool(inverse)), _ptr(x), _ptr(out), _stream(stream))
    _check("lwm_attn_rope", rc)


def lwm_attn_packed_loss_workspace_bytes(B: int, T: int, V: int, num_segments: int) -> int:
    return int(load_library().lwm_attn_packed_loss_workspace_bytes(B, T, V, num_segments))


def lwm_attn_packed_loss(logits, targets, seg, num_segments: int, loss, token_loss=None,
                         dlogits=None, workspace=None, grad_scale: float = 1.0, stream=None):
    """Reweighted packed cross-entropy of logits [B,T,V]; see include/lwm_attn.h."""
    B, T, V = logits.shape
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = load_library().lwm_attn_packed_loss(B, T, V, int(num_segments), _dtype_code(logits.dtype),
                                             _ptr(logits), _ptr(targets), _ptr(seg), float(grad_scale),
                                             _ptr(loss), _ptr(token_loss), _ptr(dlogits),
                                             _ptr(workspace), ws_bytes, _stream(stream))
    _check("lwm_attn_packed_loss", rc)


def packed_loss(logits, targets, seg, num_segments=None, *, grad=True, grad_scale=1.0, stream=None):
    """(loss, token_loss, dlogits or None) with the packed-sample reweighting."""
    import torch

    B, T, V = logits.shape
    if num_segments is None:
        num_segments = int(seg.max().item()) + 1 if seg.numel() else 1
    num_segments = max(1, num_segments)
    ws = torch.empty(max(lwm_attn_packed_loss_workspace_bytes(B, T, V, num_segments), 16),
                     dtype=torch.uint8, device=logits.device)
    loss = torch.empty(4, dtype=torch.float32, device=logits.device)  # 16 bytes, aligned
    tl = torch.empty((B, T), dtype=torch.float32, device=logits.device)
    dl = torch.empty_like(logits) if grad else None
    lwm_attn_packed_loss(logits, targets, seg, num_segments, loss, tl, dl, ws, grad_scale, stream)
    return loss[0], tl, dl


def lwm_attn_bwd_workspace_bytes(desc: Desc) -> int:
    return int(load_library().lwm_attn_bwd_workspace_bytes(ctypes.byref(desc)))


def _expect_bwd(desc, q, k, v, o, do, lse, seg_q, seg_k, table, dq, dk, dv):
    _expect_attention(desc, q, k, v, seg_q, seg_k, table,
                      qlike=(("o", o), ("dO", do), ("dQ", dq)), klike=(("dK", dk), ("dV", dv)),
                      rowf=(("lse", lse),))


def lwm_attn_bwd(desc: Desc, q, k, v, o, do, lse, seg_q, seg_k, table, dq, dk, dv, workspace,
                 stream=None):
    _expect_bwd(desc, q, k, v, o, do, lse, seg_q, seg_k, table, dq, dk, dv)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = load_library().lwm_attn_bwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                     _ptr(do), _ptr(lse), _ptr(seg_q), _ptr(seg_k), _ptr(table),
                                     _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), ws_bytes,
                                     _stream(stream))
    _check("lwm_attn_bwd", rc)


def lwm_attn_bwd_rope(desc: Desc, theta: float, q, q_rot, k, k_rot, v, o, do, lse, seg_q, seg_k,
                      table, dq, dk, dv, workspace, stream=None):
    """lwm_attn_bwd with RoPE at load: q, k unrotated, q_rot, k_rot turned; dq, dk are the
    gradients of the unrotated q, k."""
    _expect_bwd(desc, q, k, v, o, do, lse, seg_q, seg_k, table, dq, dk, dv)
    _expect_attention(desc, q_rot, k_rot)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = load_library().lwm_attn_bwd_rope(ctypes.byref(desc), float(theta), _ptr(q), _ptr(q_rot),
                                          _ptr(k), _ptr(k_rot), _ptr(v), _ptr(o), _ptr(do),
                                          _ptr(lse), _ptr(seg_q), _ptr(seg_k), _ptr(table),
                                          _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), ws_bytes,
                                          _stream(stream))
    _check("lwm_attn_bwd_rope", rc)


def lwm_attn_bwd_phase(desc: Desc, phase: int, q, k, v, o, do, lse, seg_q, seg_k, table, dq, dk,
                       dv, workspace, stream=None):
    _expect_bwd(desc, q, k, v, o, do, lse, seg_q, seg_k, table, dq, dk, dv)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = load_library().lwm_attn_bwd_phase(ctypes.byref(desc), int(phase), _ptr(q), _ptr(k),
                                           _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(seg_q),
                                           _ptr(seg_k), _ptr(table), _ptr(dq), _ptr(dk), _ptr(dv),
                                           _ptr(workspace), ws_bytes, _stream(stream))
    _check("lwm_attn_bwd_phase", rc)


# ---------------------------------------------------------------------------------------
# convenience layers (allocation with torch, then the calls above)
# ---------------------------------------------------------------------------------------

def _desc_for(q, k, *, scale, causal, q_offset, k_offset):
    B, H, Sq, D = q.shape
    Sk = k.shape[2]
    return make_desc(B, H, Sq, Sk, D, q.dtype, scale=scale, causal=causal, q_offset=q_offset,
                     k_offset=k_offset)


def rope(x, pos_offset: int, theta: float, *, inverse: bool = False, out=None, stream=None):
    """RoPE-rotated copy of x [B,H,S,D] (or into `out`, which may be x for in place)."""
    import torch

    out = torch.empty_like(x) if out is None else out
    lwm_attn_rope(x, out, pos_offset, theta, inverse, stream=stream)
    return out


def _rotated(q, k, rope_theta, q_offset, k_offset, stream):
    if rope_theta is None:
        return q, k
    return (rope(q, q_offset, rope_theta, stream=stream), rope(k, k_offset, rope_theta, stream=stream))


def _rope_at_load(q, rope_theta) -> bool:
    """RoPE inside the attention kernels' loads is built for bf16 with head width 128; other
    dtypes and widths turn Q and K with the standalone kernel first."""
    import torch

    return rope_theta is not None and q.dtype == torch.bfloat16 and q.shape[-1] == 128


def attention_forward(q, k, v, seg_q, seg_k, *, scale=None, causal=True, q_offset=0, k_offset=0,
                      table=None, rope_theta=None, stream=None):
    """(O, LSE, table) for Q [B,H,Sq,D] against K, V [B,H,Sk,D] with segment ids.  With
    rope_theta, Q and K are turned by RoPE at their global positions: K by the standalone
    kernel and Q inside the attention kernel's load (bf16, D = 128), or both first."""
    import torch

    fused = _rope_at_load(q, rope_theta)
    if fused:
        k = rope(k, k_offset, rope_theta, stream=stream)
    else:
        q, k = _rotated(q, k, rope_theta, q_offset, k_offset, stream)
    desc = _desc_for(q, k, scale=scale, causal=causal, q_offset=q_offset, k_offset=k_offset)
    if table is None:
        table = lwm_attn_build_block_table(desc, seg_q, seg_k, stream=stream)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    if fused:
        lwm_attn_fwd_rope(desc, LWM_OUT_FINAL, rope_theta, q, k, v, seg_q, seg_k, table, o=o, lse=lse,
                          stream=stream)
    else:
        lwm_attn_fwd(desc, LWM_OUT_FINAL, q, k, v, seg_q, seg_k, table, o=o, lse=lse, stream=stream)
    return o, lse, table


def attention_decode(q, k, v, seg_q, seg_k, *, scale=None, causal=True, q_offset=None,
                     k_offset=0, table=None, workspace=None, stream=None):
    """(O, LSE, table) for a few query rows against a long KV cache by split-KV decode.
    By default the queries are the cache's last Sq positions (q_offset = k_offset + Sk - Sq)."""
    import torch

    if q_offset is None:
        q_offset = k_offset + k.shape[2] - q.shape[2]
    desc = _desc_for(q, k, scale=scale, causal=causal, q_offset=q_offset, k_offset=k_offset)
    if table is None:
        table = lwm_attn_build_block_table(desc, seg_q, seg_k, stream=stream)
    if workspace is None:
        workspace = torch.empty(max(lwm_attn_decode_workspace_bytes(desc), 16), dtype=torch.uint8,
                                device=q.device)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    lwm_attn_decode(desc, q, k, v, seg_q, seg_k, table, o, lse, workspace, stream=stream)
    return o, lse, table


def attention_partial(q, k, v, seg_q, seg_k, *, scale=None, causal=True, q_offset=0, k_offset=0,
                      table=None, out=None, stream=None):
    """(m, l, acc) state of Q against one KV chunk."""
    import torch

    desc = _desc_for(q, k, scale=scale, causal=causal, q_offset=q_offset, k_offset=k_offset)
    if table is None:
        table = lwm_attn_build_block_table(desc, seg_q, seg_k, stream=stream)
    B, H, Sq, D = q.shape
    if out is None:
        m = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
        l = torch.empty_like(m)
        acc = torch.empty((B, H, Sq, D), dtype=torch.float32, device=q.device)
    else:
        m, l, acc = out
    lwm_attn_fwd(desc, LWM_OUT_PARTIAL, q, k, v, seg_q, seg_k, table, m=m, l=l, acc=acc,
                 stream=stream)
    return m, l, acc


def attention_backward(q, k, v, o, do, lse, seg_q, seg_k, table, *, scale=None, causal=True,
                       q_offset=0, k_offset=0, workspace=None, rope_theta=None, stream=None):
    """(dQ, dK, dV) by LSE recompute.  With rope_theta, q and k are the unrotated inputs of a
    RoPE forward and dQ, dK the gradients of those: for bf16 with D = 128 the kernels turn
    the operand they hold at load and turn dQ, dK back before rounding (Q and K are also
    turned once by the standalone kernel, for the operand each kernel streams); otherwise Q
    and K are turned first and dQ, dK turned back after (in place)."""
    import torch

    if _rope_at_load(q, rope_theta):
        desc = _desc_for(q, k, scale=scale, causal=causal, q_offset=q_offset, k_offset=k_offset)
        if workspace is None:
            workspace = torch.empty(max(lwm_attn_bwd_workspace_bytes(desc), 16), dtype=torch.uint8,
                                    device=q.device)
        q_rot, k_rot = _rotated(q, k, rope_theta, q_offset, k_offset, stream)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        lwm_attn_bwd_rope(desc, rope_theta, q, q_rot, k, k_rot, v, o, do, lse, seg_q, seg_k, table,
                          dq, dk, dv, workspace, stream=stream)
        return dq, dk, dv
    q, k = _rotated(q, k, rope_theta, q_offset, k_offset, stream)
    desc = _desc_for(q, k, scale=scale, causal=causal, q_offset=q_offset, k_offset=k_offset)
    if workspace is None:
        workspace = torch.empty(max(lwm_attn_bwd_workspace_bytes(desc), 16), dtype=torch.uint8,
                                device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    lwm_attn_bwd(desc, q, k, v, o, do, lse, seg_q, seg_k, table, dq, dk, dv, workspace,
                 stream=stream)
    if rope_theta is not None:
        rope(dq, q_offset, rope_theta, inverse=True, out=dq, stream=stream)
        rope(dk, k_offset, rope_theta, inverse=True, out=dk, stream=stream)
    return dq, dk, dv


def ring_order(rank: int, n_chunks: int) -> List[int]:
    """KV chunk held by device `rank` at each ring step when chunks travel one device per
    step towards higher ranks: at step t the device holds chunk (rank - t) mod N."""
    return [(rank - t) % n_chunks for t in range(n_chunks)]


def ring_share_forward(q, k_chunks: Sequence, v_chunks: Sequence, seg_q, seg_k_chunks: Sequence,
                       *, q_offset: int, chunk_offsets: Sequence[int], order: Sequence[int],
                       scale=None, causal=True, tables=None, states=None, stream=None):
    """One device's share of the ring: the query chunk Q (global offset q_offset) merged
    against the KV chunks in `order`.  Chunks whose keys all lie after the last query are
    skipped on the host (they contribute nothing under the causal mask).  The first
    contributing chunk writes the running state; each later one writes a chunk state that
    lwm_attn_merge_chunk folds in; the last merge finalises into (O, LSE).

    `tables` (optional) maps chunk index -> prebuilt table; `states` (optional) is a pair
    of preallocated (m, l, acc) triples.  Returns (O, LSE, tables)."""
    import torch

    B, H, Sq, D = q.shape
    last_q = q_offset + Sq - 1
    live = [c for c in order if not (causal and chunk_offsets[c] > last_q)]
    tables = {} if tables is None else tables
    if states is None:
        mk = lambda: (torch.empty((B, H, Sq), dtype=torch.float32, device=q.device),
                      torch.empty((B, H, Sq), dtype=torch.float32, device=q.device),
                      torch.empty((B, H, Sq, D), dtype=torch.float32, device=q.device))
        states = (mk(), mk())
    run, chunk = states
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    rows = B * H * Sq
    odt = _dtype_code(q.dtype)
    if not live:
        # every chunk is in the future: empty state finalises to O = 0, LSE = -inf
        run[0].fill_(float("-inf"))
        run[1].zero_()
        run[2].zero_()
        lwm_attn_merge_chunk(rows, D, *run, finalize=True, out_dtype=odt, o=o, lse=lse,
                             stream=stream)
        return o, lse, tables
    for step, c in enumerate(live):
        desc = _desc_for(q, k_chunks[c], scale=scale, causal=causal, q_offset=q_offset,
                         k_offset=chunk_offsets[c])
        if c not in tables:
            tables[c] = lwm_attn_build_block_table(desc, seg_q, seg_k_chunks[c], stream=stream)
        dst = run if step == 0 else chunk
        lwm_attn_fwd(desc, LWM_OUT_PARTIAL, q, k_chunks[c], v_chunks[c], seg_q, seg_k_chunks[c],
                     tables[c], m=dst[0], l=dst[1], acc=dst[2], stream=stream)
        last = step == len(live) - 1
        if step > 0:
            lwm_attn_merge_chunk(rows, D, *run, *chunk, finalize=last, out_dtype=odt, o=o,
                                 lse=lse, stream=stream)
        elif last:
            lwm_attn_merge_chunk(rows, D, *run, finalize=True, out_dtype=odt, o=o, lse=lse,
                                 stream=stream)
    return o, lse, tables
