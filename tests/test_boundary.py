"""Host-side checks of the C-ABI library: it loads, exports every entry point that
include/lwm_attn.h declares, sizes its buffers as documented, and rejects bad arguments
with the documented status codes before anything reaches a GPU (no compute call is made)."""
import ctypes
import os
import re

import pytest

import long_context_exact_blockwise_amd as lwm
from long_context_exact_blockwise_amd import build as lwm_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lwm_attn.h")

OK, INVALID, SHAPE, ALIGN, UNSUP, WS = 0, -1, -2, -3, -4, -5
FAKE = 1 << 40  # 16-byte aligned fake device address; never dereferenced by these tests


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(lwm.LIB_PATH):
        lwm_build.build()
    return lwm.load_library()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lwm_attn_\w+)\s*\(", text)))


def test_header_declares_the_four_calls_and_size_queries():
    names = header_functions()
    for n in ("lwm_attn_fwd", "lwm_attn_bwd", "lwm_attn_merge_chunk", "lwm_attn_build_block_table",
              "lwm_attn_block_table_bytes", "lwm_attn_bwd_workspace_bytes"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in header_functions():
        assert hasattr(lib, name), name
    assert set(header_functions()) == set(lwm.EXPORTED)


def test_library_is_built_for_gfx950_only():
    data = open(lwm.LIB_PATH, "rb").read()
    assert b"gfx950" in data
    for other in (b"gfx942", b"gfx90a", b"gfx1100"):
        assert b"amdgcn-amd-amdhsa--" + other not in data


def desc(**kw):
    base = dict(B=1, H=2, Sq=256, Sk=256, D=128, dtype=lwm.LWM_BF16)
    base.update(kw)
    return lwm.make_desc(base.pop("B"), base.pop("H"), base.pop("Sq"), base.pop("Sk"),
                         base.pop("D"), base.pop("dtype"), **base)


def test_status_strings(lib):
    for code in (OK, INVALID, SHAPE, ALIGN, UNSUP, WS, -6):
        s = lib.lwm_attn_status_string(code).decode()
        assert s.startswith(lwm.STATUS[code])
    assert lib.lwm_attn_status_string(-99).decode() == "LWM_ERR_UNKNOWN"
    assert lib.lwm_attn_version() >= 100


def test_table_bytes_follow_documented_layout(lib):
    def al(x):
        return (x + 255) // 256 * 256

    for (B, Sq, Sk, bq, bk) in [(1, 256, 256, 64, 64), (2, 1000, 333, 32, 16), (1, 131072, 1048576, 64, 64)]:
        d = desc(B=B, Sq=Sq, Sk=Sk, block_q=bq, block_k=bk)
        nqb, nkb = -(-Sq // bq), -(-Sk // bk)
        expect = al(B * nqb * 8) + al(B * nkb * 8) + al(B * nqb * nkb) + al(B * nqb * 16) + al(B * nkb * 16)
        assert lwm.lwm_attn_block_table_bytes(d) == expect
    assert lwm.lwm_attn_block_table_bytes(desc(block_q=48)) == 0
    assert lwm.lwm_attn_bwd_workspace_bytes(desc(B=2, H=3, Sq=100)) == 2 * al(2 * 3 * 100 * 4)


def call_fwd(lib, d, mode=0, q=FAKE, k=FAKE, v=FAKE, sq=FAKE, sk=FAKE, t=FAKE, o=FAKE, lse=FAKE,
             m=None, l=None, acc=None):
    return lib.lwm_attn_fwd(ctypes.byref(d), mode, q, k, v, sq, sk, t, o, lse, m, l, acc, None)


def test_fwd_rejects_bad_arguments(lib):
    assert lib.lwm_attn_fwd(None, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None,
                            None, None) == INVALID
    assert call_fwd(lib, desc(D=96)) == UNSUP
    assert call_fwd(lib, desc(D=64)) == UNSUP                       # bf16 needs D = 128
    assert call_fwd(lib, desc(D=128, dtype=lwm.LWM_F32)) == UNSUP   # f32 built for 32, 64
    assert call_fwd(lib, desc(block_q=32)) == UNSUP
    assert call_fwd(lib, desc(block_q=40)) == INVALID
    assert call_fwd(lib, desc(scale=-1.0)) == INVALID
    assert call_fwd(lib, desc(Sq=-1)) == SHAPE
    assert call_fwd(lib, desc(q_offset=-5)) == SHAPE
    assert call_fwd(lib, desc(), mode=7) == INVALID
    assert call_fwd(lib, desc(), q=None) == INVALID
    assert call_fwd(lib, desc(), o=None) == INVALID
    assert call_fwd(lib, desc(), mode=1) == INVALID                 # PARTIAL needs m, l, acc
    assert call_fwd(lib, desc(), q=FAKE + 8) == ALIGN
    assert call_fwd(lib, desc(), lse=FAKE + 4) == ALIGN
    # no query rows: nothing to do, succeeds without touching any pointer
    assert call_fwd(lib, desc(Sq=0), q=None, k=None, v=None, sq=None, sk=None, t=None, o=None,
                    lse=None) == OK
    d = desc()
    d.causal = 2
    assert call_fwd(lib, d) == INVALID
    d = desc()
    d.dtype = 9
    assert call_fwd(lib, d) == INVALID


def test_table_builder_rejects_bad_arguments(lib):
    f = lib.lwm_attn_build_block_table
    assert f(ctypes.byref(desc()), None, FAKE, FAKE, None) == INVALID
    assert f(ctypes.byref(desc()), FAKE, FAKE, FAKE + 2, None) == ALIGN
    assert f(ctypes.byref(desc(block_k=128)), FAKE, FAKE, FAKE, None) == INVALID
    assert f(ctypes.byref(desc(B=0)), FAKE, FAKE, FAKE, None) == SHAPE


def test_merge_rejects_bad_arguments(lib):
    f = lib.lwm_attn_merge_chunk
    args = lambda **kw: [kw.get(n, FAKE) for n in ("m", "l", "acc", "mc", "lc", "accc")]
    assert f(10, 130, *args(), 0, 0, None, None, None) == SHAPE       # D % 4
    assert f(10, 512, *args(), 0, 0, None, None, None) == SHAPE       # D > 256
    assert f(-1, 128, *args(), 0, 0, None, None, None) == SHAPE
    assert f(10, 128, *args(), 2, 0, None, None, None) == INVALID     # finalize flag
    assert f(10, 128, *args(), 0, 5, None, None, None) == INVALID     # out dtype
    assert f(10, 128, *args(lc=None), 0, 0, None, None, None) == INVALID   # partial chunk
    assert f(10, 128, *args(mc=None, lc=None, accc=None), 0, 0, None, None, None) == INVALID
    assert f(10, 128, *args(), 1, 0, None, FAKE, None) == INVALID     # finalize needs o
    assert f(10, 128, *args(acc=FAKE + 4), 0, 0, None, None, None) == ALIGN
    assert f(0, 128, *args(), 0, 0, None, None, None) == OK           # no rows


def test_bwd_rejects_bad_arguments(lib):
    f = lib.lwm_attn_bwd

    def call(d, ws=FAKE, ws_bytes=1 << 30, **kw):
        names = ("q", "k", "v", "o", "do", "lse", "sq", "sk", "t", "dq", "dk", "dv")
        return f(ctypes.byref(d), *[kw.get(n, FAKE) for n in names], ws, ws_bytes, None)

    assert call(desc(D=64)) == UNSUP
    assert call(desc(), do=None) == INVALID
    assert call(desc(), ws=None) == WS
    assert call(desc(), ws_bytes=16) == WS
    assert call(desc(), dk=FAKE + 2) == ALIGN
    assert call(desc(Sq=0, Sk=0)) == OK


def test_bwd_phase_rejects_bad_phase(lib):
    f = lib.lwm_attn_bwd_phase
    args = [FAKE] * 12
    assert f(ctypes.byref(desc()), 3, *args, FAKE, 1 << 30, None) == INVALID
    assert f(ctypes.byref(desc()), -1, *args, FAKE, 1 << 30, None) == INVALID
    assert f(ctypes.byref(desc(D=64)), 1, *args, FAKE, 1 << 30, None) == UNSUP


def test_decode_workspace_size(lib):
    def al(x):
        return (x + 255) // 256 * 256

    # one new token per head against a 1M-token cache: the slices' states take a few MiB
    for (H, Sq, Sk) in [(32, 1, 1 << 20), (32, 16, 1 << 20), (8, 4, 5000), (2, 300, 777), (1, 1, 0)]:
        n = lwm.lwm_attn_decode_workspace_bytes(desc(H=H, Sq=Sq, Sk=Sk))
        rows = H * Sq
        # layout m [ns][rows], l [ns][rows], acc [ns][rows][128] for some slice count ns
        ns = [s for s in range(1, 65536) if 2 * al(s * rows * 4) + al(s * rows * 512) == n]
        assert ns, (H, Sq, Sk, n)
        ntiles = -(-Sk // 64)
        assert ns[0] <= max(1, ntiles)
        if Sk == 1 << 20:
            assert ns[0] >= 64
            assert n < (8 << 20 if Sq == 1 else 128 << 20)
    assert lwm.lwm_attn_decode_workspace_bytes(desc(dtype=lwm.LWM_F32, D=64)) == 0
    assert lwm.lwm_attn_decode_workspace_bytes(desc(block_q=32)) == 0
    assert lwm.lwm_attn_decode_workspace_bytes(desc(Sq=0)) == 0


def test_decode_rejects_bad_arguments(lib):
    f = lib.lwm_attn_decode

    def call(d, ws=FAKE, ws_bytes=1 << 30, **kw):
        names = ("q", "k", "v", "sq", "sk", "t", "o", "lse")
        return f(ctypes.byref(d), *[kw.get(n, FAKE) for n in names], ws, ws_bytes, None)

    assert call(desc(D=64, dtype=lwm.LWM_F32)) == UNSUP
    assert call(desc(D=64)) == UNSUP
    assert call(desc(block_k=32)) == UNSUP
    assert call(desc(scale=0.0)) == INVALID
    assert call(desc(), o=None) == INVALID
    assert call(desc(), t=None) == INVALID
    assert call(desc(), ws=None) == WS
    assert call(desc(), ws_bytes=lwm.lwm_attn_decode_workspace_bytes(desc()) - 1) == WS
    assert call(desc(), v=FAKE + 8) == ALIGN
    assert call(desc(), ws=FAKE + 4) == ALIGN
    assert call(desc(Sq=0), q=None, k=None, v=None, sq=None, sk=None, t=None, o=None, lse=None,
                ws=None, ws_bytes=0) == OK


def test_decode_noalloc_rejects_bad_arguments_and_oversize(lib):
    f = lib.lwm_attn_decode_noalloc

    def call(d, **kw):
        names = ("q", "k", "v", "sq", "sk", "t", "o", "lse")
        return f(ctypes.byref(d), *[kw.get(n, FAKE) for n in names], None)

    assert lwm.DECODE_SCRATCH_BYTES == 64 << 20
    assert call(desc(D=64, dtype=lwm.LWM_F32)) == UNSUP
    assert call(desc(block_k=32)) == UNSUP
    assert call(desc(scale=0.0)) == INVALID
    assert call(desc(), o=None) == INVALID
    assert call(desc(), lse=None) == INVALID
    assert call(desc(), v=FAKE + 8) == ALIGN
    # one slice state per query row: B*H*Sq*(D+2)*4 bytes (plus three 256-byte alignments)
    # must fit the 64 MiB buffer; 129000 rows fit, 129100 do not; rejected on the host
    fits = (lwm.DECODE_SCRATCH_BYTES - 3 * 256) // (130 * 4)
    assert call(desc(H=1, Sq=fits + 1, Sk=4096)) == WS
    assert call(desc(B=2, H=32, Sq=4096, Sk=1 << 20)) == WS
    assert call(desc(Sq=0), q=None, k=None, v=None, sq=None, sk=None, t=None, o=None,
                lse=None) == OK


def test_rope_rejects_bad_arguments(lib):
    f = lib.lwm_attn_rope

    def call(B=1, H=2, S=100, D=128, dtype=lwm.LWM_BF16, pos=0, theta=1e6, inverse=0, x=FAKE,
             out=FAKE):
        return f(B, H, S, D, dtype, pos, theta, inverse, x, out, None)

    assert call(D=96) == UNSUP
    assert call(D=512) == UNSUP
    assert call(dtype=7) == INVALID
    assert call(inverse=2) == INVALID
    assert call(theta=1.0) == INVALID
    assert call(theta=float("nan")) == INVALID
    assert call(theta=float("inf")) == INVALID
    assert call(S=-1) == SHAPE
    assert call(pos=-3) == SHAPE
    assert call(pos=(1 << 32) - 99) == SHAPE          # last position 2^32 is out of range
    assert call(x=None) == INVALID
    assert call(out=FAKE + 8) == ALIGN
    assert call(out=FAKE + 256) == INVALID           # partial overlap with x
    assert call(S=0, x=None, out=None) == OK         # nothing to do


def test_packed_loss_workspace_and_rejections(lib):
    def al(x):
        return (x + 255) // 256 * 256

    assert lwm.lwm_attn_packed_loss_workspace_bytes(2, 1000, 40192, 30) == al(2 * 30 * 4) + 256 + al(2 * 1000 * 4)
    assert lwm.lwm_attn_packed_loss_workspace_bytes(1, 10, 12, 1) == 0      # V % 8
    assert lwm.lwm_attn_packed_loss_workspace_bytes(1, 10, 16, 0) == 0      # no segment
    f = lib.lwm_attn_packed_loss

    def call(B=1, T=100, V=40192, nseg=4, dtype=lwm.LWM_BF16, g=1.0, logits=FAKE, tg=FAKE, seg=FAKE,
             loss=FAKE, tl=None, dl=FAKE, ws=FAKE, ws_bytes=1 << 30):
        return f(B, T, V, nseg, dtype, logits, tg, seg, g, loss, tl, dl, ws, ws_bytes, None)

    assert call(V=100) == UNSUP
    assert call(V=262144) == UNSUP
    assert call(V=131072, dtype=lwm.LWM_F32) == UNSUP
    assert call(nseg=0) == SHAPE
    assert call(T=-1) == SHAPE
    assert call(dtype=5) == INVALID
    assert call(g=float("nan")) == INVALID
    assert call(loss=None) == INVALID
    assert call(seg=None) == INVALID
    assert call(ws=None) == WS
    assert call(ws_bytes=100) == WS
    assert call(dl=FAKE + 2) == ALIGN


def test_header_is_plain_c(tmp_path):
    """include/lwm_attn.h is a C header: it compiles as C99 with warnings as errors."""
    import shutil
    import subprocess

    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "use_header.c"
    src.write_text('#include "lwm_attn.h"\n'
                   "int main(void) { lwm_attn_desc d = {0}; (void)d;\n"
                   "  return lwm_attn_version() > 0 ? 0 : 1; }\n")
    r = subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-fsyntax-only",
                        "-I", os.path.join(ROOT, "include"), str(src)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_python_wrappers_check_buffer_sizes():
    """The binding raises before any pointer reaches the library when a buffer does not match
    the desc: a wrong element count or dtype, or a table built for a smaller problem (CPU
    tensors: the size check comes before the device check)."""
    torch = pytest.importorskip("torch")
    d = desc(B=1, H=2, Sq=100, Sk=120)
    bf = torch.bfloat16
    q = torch.zeros((1, 2, 100, 128), dtype=bf)
    k = torch.zeros((1, 2, 120, 128), dtype=bf)
    sq = torch.zeros((1, 100), dtype=torch.int32)
    sk = torch.zeros((1, 120), dtype=torch.int32)
    tab = torch.zeros(lwm.lwm_attn_block_table_bytes(d), dtype=torch.uint8)
    o = torch.zeros_like(q)
    lse = torch.zeros((1, 2, 100), dtype=torch.float32)
    ok = dict(q=q, k=k, v=k, seg_q=sq, seg_k=sk, table=tab, o=o, lse=lse)

    def fwd(**kw):
        a = {**ok, **kw}
        lwm.lwm_attn_fwd(d, lwm.LWM_OUT_FINAL, a["q"], a["k"], a["v"], a["seg_q"], a["seg_k"],
                         a["table"], o=a["o"], lse=a["lse"])

    with pytest.raises(ValueError, match="tensors must live on the GPU"):
        fwd()                                   # every size right: only the device check fails
    with pytest.raises(ValueError, match="k has"):
        fwd(k=torch.zeros((1, 2, 100, 128), dtype=bf))
    with pytest.raises(ValueError, match="dtype"):
        fwd(v=k.float())
    with pytest.raises(ValueError, match="o has"):
        fwd(o=torch.zeros((1, 2, 99, 128), dtype=bf))
    with pytest.raises(ValueError, match="lse has"):
        fwd(lse=torch.zeros((1, 2, 128), dtype=torch.float32))
    with pytest.raises(ValueError, match="seg_k"):
        fwd(seg_k=torch.zeros((1, 100), dtype=torch.int32))
    with pytest.raises(ValueError, match="table"):
        fwd(table=tab[: tab.numel() - 256])
    dq, dk = torch.zeros_like(q), torch.zeros_like(k)
    with pytest.raises(ValueError, match="dV has"):
        lwm.lwm_attn_bwd(d, q, k, k, o, o, lse, sq, sk, tab, dq, dk, torch.zeros_like(q), None)
    with pytest.raises(ValueError, match="dO has"):
        lwm.lwm_attn_bwd_phase(d, lwm.LWM_BWD_DQ, q, k, k, o, k, lse, sq, sk, tab, dq, dk, dk, None)
    with pytest.raises(ValueError, match="lse has"):
        lwm.lwm_attn_decode(d, q, k, k, sq, sk, tab, o, lse[:, :1], None)
    with pytest.raises(ValueError, match="o has"):
        lwm.lwm_attn_decode_noalloc(d, q, k, k, sq, sk, tab, k, lse)


def test_rope_at_load_rejects_bad_arguments(lib):
    fwd, bwd = lib.lwm_attn_fwd_rope, lib.lwm_attn_bwd_rope

    def cf(d, theta=1e6, mode=0, **kw):
        names = ("q", "k", "v", "sq", "sk", "t", "o", "lse", "m", "l", "acc")
        return fwd(ctypes.byref(d), mode, theta, *[kw.get(n, FAKE) for n in names], None)

    def cb(d, theta=1e6, ws_bytes=1 << 30, **kw):
        names = ("q", "qr", "k", "kr", "v", "o", "do", "lse", "sq", "sk", "t", "dq", "dk", "dv", "ws")
        return bwd(ctypes.byref(d), theta, *[kw.get(n, FAKE) for n in names], ws_bytes, None)

    for call in (cf, cb):
        assert call(desc(D=64, dtype=lwm.LWM_F32)) == UNSUP   # RoPE at load: bf16, D = 128
        assert call(desc(D=64)) == UNSUP
        assert call(desc(), theta=1.0) == INVALID
        assert call(desc(), theta=float("inf")) == INVALID
        assert call(desc(q_offset=(1 << 32) - 255)) == SHAPE    # positions beyond 2^32
        assert call(desc(k_offset=(1 << 32) - 100)) == SHAPE
    assert cf(desc(), mode=2) == INVALID
    assert cf(desc(), k=None) == INVALID
    assert cf(desc(), v=FAKE + 8) == ALIGN
    assert cb(desc(), qr=None) == INVALID
    assert cb(desc(), kr=FAKE + 4) == ALIGN
    assert cb(desc(), ws=None) == WS
    assert cb(desc(), ws_bytes=lwm.lwm_attn_bwd_workspace_bytes(desc()) - 1) == WS


def test_debug_status_in_normal_and_debug_builds(lib):
    """The normal build has no device checks (LWM_ERR_UNSUPPORTED, words zeroed); both builds
    reject a NULL words pointer and unknown flags before any HIP call.  The debug build
    exports the same symbols."""
    w = (ctypes.c_uint32 * 2)(7, 7)
    assert lib.lwm_attn_debug_status(w, 0) == UNSUP
    assert list(w) == [0, 0]
    assert lib.lwm_attn_debug_status(None, 0) == INVALID
    if not os.path.exists(lwm.DEBUG_LIB_PATH):
        lwm_build.build()
    dbg = lwm._open_library(lwm.DEBUG_LIB_PATH)
    for name in header_functions():
        assert hasattr(dbg, name), name
    assert dbg.lwm_attn_debug_status(None, 0) == INVALID
    assert dbg.lwm_attn_debug_status(w, 2) == INVALID
    assert dbg.lwm_attn_debug_status(w, -1) == INVALID
    # argument checks are the same code in both builds
    d = desc()
    assert dbg.lwm_attn_fwd(ctypes.byref(d), 0, None, None, None, None, None, None, None, None,
                            None, None, None, None) == INVALID


def test_missing_library_fails_loudly(tmp_path):
    """With no built library the package raises on the first call; there is no fallback."""
    import subprocess
    import sys

    code = ("import long_context_exact_blockwise_amd as lwm\n"
            "d = lwm.make_desc(1, 1, 64, 64, 128, lwm.LWM_BF16)\n"
            "try:\n"
            "    lwm.lwm_attn_block_table_bytes(d)\n"
            "except RuntimeError as e:\n"
            "    print('raised:', e)\n"
            "    raise SystemExit(0)\n"
            "raise SystemExit(3)\n")
    env = dict(os.environ, LWM_ATTN_LIBRARY=str(tmp_path / "absent.so"))
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "not built" in r.stdout
