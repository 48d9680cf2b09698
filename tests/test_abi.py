"""The C-ABI library on the host: it loads, exports what include/*.h declare,
and rejects bad arguments before touching the GPU. No kernel runs here."""
import ctypes
import glob
import os
import re
import subprocess

import numpy as np
import pytest

import paged_kv_cache_slot_amd as pa
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))

PA_OK, PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE = 0, -1, -2, -3, -4


def declared_functions():
    names = set()
    for header in HEADERS:
        with open(header) as f:
            text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
        names |= set(re.findall(r"\b(pa_[a-z_0-9]+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pa.lib_path):
        pytest.fail("libpa.so is not built (run __graft_entry__.build())")
    return pa.library()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(pa.EXPORTED_SYMBOLS)
    out = subprocess.run(["nm", "-D", "--defined-only", pa.lib_path], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (pa_\w+)", out))
    assert set(names) <= exported, set(names) - exported
    for n in names:
        assert getattr(lib, n) is not None


def test_status_strings(lib):
    for code in (PA_OK, PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE, -5, -6, -7,
                 -8):
        assert pa.pa_status_string(code) not in ("", "unknown status")
    assert pa.pa_status_string(1234) == "unknown status"


def _fake(addr=0x10000):
    return ctypes.c_void_p(addr)   # never dereferenced: every call below fails a host check


def test_store_argument_checks(lib):
    f = lib.pa_store_kvcache
    P = _fake()
    assert f(None, None, 1024, None, None, None, 0, 10, 256, 8, 128, None) == PA_OK  # nothing to do
    assert f(P, P, 1024, P, P, None, 4, 10, 256, 8, 128, None) == PA_ERR_NULL
    assert f(P, P, 1024, P, P, P, -1, 10, 256, 8, 128, None) == PA_ERR_SHAPE
    assert f(P, P, 1000, P, P, P, 4, 10, 256, 8, 128, None) == PA_ERR_SHAPE  # stride < row
    assert f(P, P, 512, P, P, P, 4, 10, 256, 8, 64, None) == PA_ERR_UNSUPPORTED  # head_dim
    assert f(P, P, 1024, P, P, P, 4, 10, 100, 8, 128, None) == PA_ERR_UNSUPPORTED  # block size
    assert f(P, P, 1028, P, P, P, 4, 10, 256, 8, 128, None) == PA_ERR_UNSUPPORTED  # stride % 8
    assert f(_fake(0x10002), P, 1024, P, P, P, 4, 10, 256, 8, 128, None) == PA_ERR_UNSUPPORTED


def test_decode_argument_checks(lib):
    f = lib.pa_decode
    P = _fake()
    ws = pa.pa_decode_workspace_bytes(4, 16, 128, 300, 256)
    base = dict(out=P, q=P, kc=P, vc=P, bt=P, stride=2, cl=P, B=4, hq=16, hkv=8, d=128, bs=256,
                maxl=300, scale=0.088, ws=P, wsb=ws)

    def call(**kw):
        a = dict(base, **kw)
        return f(a["out"], a["q"], a["kc"], a["vc"], a["bt"], a["stride"], a["cl"], a["B"],
                 a["hq"], a["hkv"], a["d"], a["bs"], a["maxl"], a["scale"], a["ws"], a["wsb"], None)

    assert call(B=0) == PA_OK
    assert call(q=None) == PA_ERR_NULL
    assert call(hq=12) == PA_ERR_SHAPE            # 12 % 8 != 0
    assert call(hq=24, hkv=8) == PA_ERR_UNSUPPORTED  # G = 3
    assert call(hq=128, hkv=8) == PA_ERR_UNSUPPORTED  # G = 16
    assert call(d=64) == PA_ERR_UNSUPPORTED
    assert call(bs=8) == PA_ERR_UNSUPPORTED
    assert call(stride=1) == PA_ERR_SHAPE         # 1 block cannot hold 300 tokens
    assert call(wsb=ws - 1) == PA_ERR_WORKSPACE
    assert call(ws=None) == PA_ERR_WORKSPACE
    assert call(maxl=-1) == PA_ERR_SHAPE
    for bad in (0.0, -0.088, float("nan"), float("inf")):
        assert call(scale=bad) == PA_ERR_SHAPE


def test_decode_store_argument_checks(lib):
    f = lib.pa_decode_store
    P = _fake()
    ws = pa.pa_decode_workspace_bytes(4, 16, 128, 300, 256)
    base = dict(out=P, q=P, kn=P, vn=P, kvs=1024, kc=P, vc=P, sm=P, bt=P, stride=2, cl=P, B=4,
                nb=10, hq=16, hkv=8, d=128, bs=256, maxl=300, scale=0.088, ws=P, wsb=ws)

    def call(**kw):
        a = dict(base, **kw)
        return f(a["out"], a["q"], a["kn"], a["vn"], a["kvs"], a["kc"], a["vc"], a["sm"], a["bt"],
                 a["stride"], a["cl"], a["B"], a["nb"], a["hq"], a["hkv"], a["d"], a["bs"],
                 a["maxl"], a["scale"], a["ws"], a["wsb"], None)

    assert call(B=0) == PA_OK
    for name in ("out", "q", "kn", "vn", "kc", "vc", "sm", "bt", "cl"):
        assert call(**{name: None}) == PA_ERR_NULL, name
    assert call(kvs=1000) == PA_ERR_SHAPE          # stride < Hkv * D
    assert call(kvs=1028) == PA_ERR_UNSUPPORTED    # stride % 8
    assert call(kn=_fake(0x10002)) == PA_ERR_UNSUPPORTED
    assert call(nb=-1) == PA_ERR_SHAPE
    assert call(hq=24, hkv=8) == PA_ERR_UNSUPPORTED  # G = 3
    assert call(d=64) == PA_ERR_UNSUPPORTED
    assert call(stride=1) == PA_ERR_SHAPE          # 1 block cannot hold 300 tokens
    assert call(wsb=ws - 1) == PA_ERR_WORKSPACE
    assert call(ws=None) == PA_ERR_WORKSPACE
    for bad in (0.0, -0.088, float("nan"), float("inf")):
        assert call(scale=bad) == PA_ERR_SHAPE


def test_decode_store_noalloc_argument_checks(lib):
    f = lib.pa_decode_store_noalloc
    P = _fake()
    base = dict(out=P, q=P, kn=P, vn=P, kvs=1024, kc=P, vc=P, sm=P, bt=P, stride=2, cl=P, B=4,
                nb=10, hq=16, hkv=8, d=128, bs=256, maxl=300, scale=0.088)

    def call(**kw):
        a = dict(base, **kw)
        return f(a["out"], a["q"], a["kn"], a["vn"], a["kvs"], a["kc"], a["vc"], a["sm"], a["bt"],
                 a["stride"], a["cl"], a["B"], a["nb"], a["hq"], a["hkv"], a["d"], a["bs"],
                 a["maxl"], a["scale"], None)

    assert call(B=0) == PA_OK
    for name in ("out", "q", "kn", "vn", "kc", "vc", "sm", "bt", "cl"):
        assert call(**{name: None}) == PA_ERR_NULL, name
    assert call(kvs=1000) == PA_ERR_SHAPE
    assert call(kvs=1028) == PA_ERR_UNSUPPORTED
    assert call(hq=24, hkv=8) == PA_ERR_UNSUPPORTED
    assert call(stride=1) == PA_ERR_SHAPE
    for bad in (0.0, float("nan")):
        assert call(scale=bad) == PA_ERR_SHAPE


def test_prefill_argument_checks(lib):
    f = lib.pa_prefill_varlen
    P = _fake()
    assert f(P, P, P, P, P, P, P, 4, 0, 0, 0, 32, 8, 128, 256, 0.1, None) == PA_OK
    assert f(P, None, P, P, P, P, P, 4, 2, 10, 8, 32, 8, 128, 256, 0.1, None) == PA_ERR_NULL
    assert f(P, P, P, P, P, P, P, 4, 2, 10, 8, 32, 8, 96, 256, 0.1, None) == PA_ERR_UNSUPPORTED
    assert f(P, P, P, P, P, P, P, 4, 2, 10, 8, 30, 8, 128, 256, 0.1, None) == PA_ERR_SHAPE
    assert f(P, P, P, P, P, P, P, 0, 2, 10, 8, 32, 8, 128, 256, 0.1, None) == PA_ERR_SHAPE
    for bad in (0.0, -0.1, float("nan"), float("inf")):
        assert f(P, P, P, P, P, P, P, 4, 2, 10, 8, 32, 8, 128, 256, bad, None) == PA_ERR_SHAPE


def test_workspace_size():
    """Header (64 B) + per-wavefront record (4 int64) for nw <= t(2048) + 1
    wavefronts + 2 (t(Hq * 2048) + Hq) partial records of 132 floats, where
    t(f) = max(u // 16, min(u // 4, f)), u = rows * Hq * (ceil(L / 8) + 2),
    rows = min(batch, 1024): a wavefront takes 16 cost units, or down to 4 while
    fewer than 2048 wavefronts would work."""
    def expect(batch, hq, max_len):
        rows = min(batch, 1024)
        u = rows * hq * ((max_len + 7) // 8 + 2)
        nw = max(u // 16, min(u // 4, 2048)) + 1
        recs = max(u // 16, min(u // 4, hq * 2048)) + hq
        return 64 + nw * 32 + 2 * recs * 132 * 4
    assert pa.pa_decode_workspace_bytes(256, 16, 128, 2048, 256) == 71877216 == expect(256, 16, 2048)
    for args in ((3, 4, 0), (3, 4, 257), (1, 32, 2048), (4096, 32, 2048)):
        assert pa.pa_decode_workspace_bytes(args[0], args[1], 128, args[2], 16) == expect(*args)
    assert pa.pa_decode_workspace_bytes(4096, 32, 128, 2048, 16) == \
        pa.pa_decode_workspace_bytes(1024, 32, 128, 2048, 16)
    assert pa.pa_decode_workspace_bytes(0, 4, 128, 257, 16) == 0


@pytest.mark.parametrize("name", ["tiny_decode", "qwen3_8b_prefill_prefix"])
def test_validate_metadata_accepts_generated(name):
    case = workloads.workload_case(name, **({} if name == "tiny_decode" else dict(batch=12)))
    pa.pa_validate_metadata(case["block_table"], case["context_lens"], case["num_blocks"],
                            case["block_size"], cu_seqlens_q=case.get("cu_seqlens_q"),
                            slot_mapping=case["slot_mapping"])


def test_validate_metadata_rejects():
    case = workloads.workload_case("qwen3_8b_decode", batch=20, pad=2)
    bt = case["block_table"].numpy().copy()
    cl = case["context_lens"].numpy().copy()
    sm = case["slot_mapping"].numpy().copy()
    nb, bs = case["num_blocks"], case["block_size"]
    pa.pa_validate_metadata(bt, cl, nb, bs, slot_mapping=sm, max_context_len=int(cl.max()))
    bad = bt.copy(); bad[0, 0] = nb
    with pytest.raises(pa.PAError, match="out of"):
        pa.pa_validate_metadata(bad, cl, nb, bs)
    bad = bt.copy(); bad[1, 0] = bad[0, 0]
    with pytest.raises(pa.PAError):  # noqa: PT012 - two rows may share a block, a row may not repeat
        b2 = bt.copy(); b2[0, 1] = b2[0, 0]
        pa.pa_validate_metadata(b2, np.maximum(cl, bs + 1), nb, bs)
    pa.pa_validate_metadata(bad, cl, nb, bs)   # shared between rows: allowed (prefix caching)
    s2 = sm.copy(); s2[3] = s2[4] if s2[4] >= 0 else s2[5]
    with pytest.raises(pa.PAError, match="twice"):
        pa.pa_validate_metadata(bt, cl, nb, bs, slot_mapping=s2)
    with pytest.raises(pa.PAError, match="context_lens"):
        pa.pa_validate_metadata(bt, cl, nb, bs, max_context_len=int(cl.max()) - 1)
    cu = np.array([0, 5, 3] + [3] * 18, dtype=np.int32)
    with pytest.raises(pa.PAError, match="new tokens"):
        pa.pa_validate_metadata(bt, cl, nb, bs, cu_seqlens_q=cu)


# ------------------------------------------------------ decode-step graphs --

def test_step_buffers_layout_matches_c(tmp_path):
    """The binding's ctypes structure has the C struct's size and field offsets."""
    fields = [f for f, _ in pa._StepBuffers._fields_]
    src = tmp_path / "layout.c"
    src.write_text('#include <stddef.h>\n#include <stdio.h>\n#include "pa.h"\nint main(void) {\n'
                   '  printf("%zu\\n", sizeof(pa_decode_step_buffers));\n' +
                   "".join(f'  printf("%zu\\n", offsetof(pa_decode_step_buffers, {f}));\n'
                           for f in fields) + "  return 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", f"-I{ROOT}/include", str(src), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True,
                                          check=True).stdout.split()]
    assert got[0] == ctypes.sizeof(pa._StepBuffers)
    assert got[1:] == [getattr(pa._StepBuffers, f).offset for f in fields]


def _step_buffers(**kw):
    P = 0x10000
    base = dict(out=P, q=P, k_new=P, v_new=P, kv_token_stride=1024, k_cache=P, v_cache=P,
                slot_mapping=P, context_lens=P, block_table=P, block_table_stride=8,
                workspace=P, workspace_bytes=pa.pa_decode_workspace_bytes(512, 16, 128, 2048, 256),
                num_blocks=100, block_size=256, num_q_heads=16, num_kv_heads=8, head_dim=128,
                max_context_len=2048, scale=0.088)
    base.update(kw)
    return pa._StepBuffers(**base)


def test_decode_graphs_argument_checks(lib):
    """Every failing check returns before any HIP call (nothing here reaches the GPU)."""
    f = lib.pa_decode_graphs_create
    h = ctypes.c_void_p(123)

    def create(buckets=None, **kw):
        arr = (ctypes.c_int32 * len(buckets))(*buckets) if buckets else None
        return f(ctypes.byref(_step_buffers(**kw)), arr, len(buckets or []), ctypes.byref(h))

    assert f(None, None, 0, ctypes.byref(h)) == PA_ERR_NULL and h.value is None
    assert f(ctypes.byref(_step_buffers()), None, 0, None) == PA_ERR_NULL
    assert create(buckets=[1, 2, 2]) == PA_ERR_SHAPE          # not increasing
    assert create(buckets=[0, 4]) == PA_ERR_SHAPE
    assert f(ctypes.byref(_step_buffers()), (ctypes.c_int32 * 1)(4), 0,
             ctypes.byref(h)) == PA_ERR_SHAPE                   # empty bucket list
    assert create(scale=0.0) == PA_ERR_SHAPE
    assert create(num_q_heads=24) == PA_ERR_UNSUPPORTED        # G = 3
    assert create(block_size=8) == PA_ERR_UNSUPPORTED
    assert create(block_table_stride=7) == PA_ERR_SHAPE        # 7 * 256 < 2048
    assert create(kv_token_stride=1000) == PA_ERR_SHAPE
    assert create(kv_token_stride=1028) == PA_ERR_UNSUPPORTED
    assert create(q=None) == PA_ERR_NULL
    assert create(out=0x10002) == PA_ERR_UNSUPPORTED
    # the default buckets end at 512 rows, so 512 rows of workspace are needed
    assert create(workspace_bytes=pa.pa_decode_workspace_bytes(256, 16, 128, 2048, 256)) == \
        PA_ERR_WORKSPACE
    assert create(buckets=[1, 256], workspace=None) == PA_ERR_WORKSPACE
    b = ctypes.c_int32()
    assert lib.pa_decode_graphs_bucket(None, 4, ctypes.byref(b)) == PA_ERR_NULL
    assert lib.pa_decode_graphs_launch(None, 4, None) == PA_ERR_NULL
    lib.pa_decode_graphs_destroy(None)


def test_sample_argument_checks(lib):
    f = lib.pa_sample_gumbel
    P = _fake()
    ws = pa.pa_sample_workspace_bytes(4, 1000)
    assert ws == 4 * 1 * 8                                 # one tile per row, one chunk
    assert pa.pa_sample_workspace_bytes(256, 151936) == 256 * 8 * 8
    assert pa.pa_sample_workspace_bytes(1, 151936) == 149 * 8
    assert f(P, P, 1000, 0, 1000, 1, 2, None, 0, None) == PA_OK        # empty batch
    assert f(P, P, 1000, 4, 0, 1, 2, P, ws, None) == PA_ERR_SHAPE      # empty vocabulary
    assert f(P, P, 996, 4, 1000, 1, 2, P, ws, None) == PA_ERR_SHAPE    # stride < vocab
    assert f(P, P, 1000, 70000, 1000, 1, 2, P, ws, None) == PA_ERR_UNSUPPORTED
    assert f(None, P, 1000, 4, 1000, 1, 2, P, ws, None) == PA_ERR_NULL
    assert f(P, _fake(0x10002), 1000, 4, 1000, 1, 2, P, ws, None) == PA_ERR_UNSUPPORTED
    assert f(P, P, 1000, 4, 1000, 1, 2, P, ws - 1, None) == PA_ERR_WORKSPACE
    assert f(P, P, 1000, 4, 1000, 1, 2, None, ws, None) == PA_ERR_WORKSPACE
