"""CPU checks of the knob surface: moe_knob_cache_lookup (a host-only text
lookup, no GPU involved), the host-side validation of moe_forward_knobs, and
the knob cache shipped with the package.  The pages resolve knobs once per
buffer capacity: a persistent cache first, then a default heuristic, with no
compilation [MegaMoE drop workflow, §6]."""
import ctypes
import os

import pytest

import mixture_experts_layer_sort_amd as lib

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, -1, -2, -3
FAKE = 0x1000  # never dereferenced: every call below returns before enqueueing

LINE = "mxfp8 swiglu 7168 2048 256 8 4096 16384 : 3 1 2048 0 5 2\n"


def _shape(H=7168, I=2048, E=256, k=8, T=8192, dt="mxfp8", act="swiglu"):
    return lib.make_shape(H, I, E, k, T, dt, act)


def _write(tmp_path, text, name="knobs.txt"):
    p = tmp_path / name
    p.write_text(text)
    return str(p)


def test_default_knobs():
    assert lib.moe_default_knobs().as_dict() == {"gemm": 0, "down_fp8": 1, "band_rows": 0, "fc2_reduce": 0,
                                                 "blocks_per_cu": 0, "load_balance": 0}


def test_missing_file_gives_defaults(tmp_path):
    kn, found = lib.moe_knob_cache_lookup(_shape(), 8192, path=str(tmp_path / "absent.txt"))
    assert not found and kn.as_dict() == lib.moe_default_knobs().as_dict()


def test_matching_line_and_token_range(tmp_path):
    path = _write(tmp_path, "# a comment line\n\n" + LINE)
    for T, hit in ((4095, False), (4096, True), (8192, True), (16384, True), (16385, False)):
        kn, found = lib.moe_knob_cache_lookup(_shape(), T, path=path)
        assert found == hit, T
        if hit:
            assert kn.as_dict() == {"gemm": 3, "down_fp8": 1, "band_rows": 2048, "fc2_reduce": 0, "blocks_per_cu": 5,
                                    "load_balance": 2}
        else:
            assert kn.as_dict() == lib.moe_default_knobs().as_dict()


@pytest.mark.parametrize("field,value", [("H", 4096), ("I", 1024), ("E", 128), ("k", 6), ("dt", "nvfp4"),
                                         ("dt", "bf16_mxfp8"), ("act", "relu2")])
def test_every_shape_field_is_part_of_the_key(tmp_path, field, value):
    path = _write(tmp_path, LINE)
    kw = {field: value}
    if field == "act":
        kw["dt"] = "mxfp8"
    _, found = lib.moe_knob_cache_lookup(_shape(**kw), 8192, path=path)
    assert not found


def test_first_matching_line_wins_and_comments_are_ignored(tmp_path):
    text = ("bf16 swiglu 7168 2048 256 8 0 100000 : 1 1 0 0 0 0\n"      # other dtype
            "mxfp8 swiglu 7168 2048 256 8 1 4095 : 1 1 0 0 4 0   # small T\n"
            "mxfp8 swiglu 7168 2048 256 8 4096 9000 : 3 0 512 1 0 1\n"
            "mxfp8 swiglu 7168 2048 256 8 0 100000 : 2 1 0 0 0 0\n")
    path = _write(tmp_path, text)
    assert lib.moe_knob_cache_lookup(_shape(), 64, path=path)[0].as_dict()["gemm"] == 1
    kn, found = lib.moe_knob_cache_lookup(_shape(), 8192, path=path)
    assert found and kn.as_dict() == {"gemm": 3, "down_fp8": 0, "band_rows": 512, "fc2_reduce": 1, "blocks_per_cu": 0,
                                      "load_balance": 1}
    assert lib.moe_knob_cache_lookup(_shape(), 9001, path=path)[0].as_dict()["gemm"] == 2


@pytest.mark.parametrize("bad", [
    "mxfp8 swiglu 7168 2048 256 8 4096 16384 3 1 2048 0 0 0\n",      # no ':'
    "mxfp8 swiglu 7168 2048 256 8 4096 16384 : 3 1 2048 0 0\n",      # a knob missing
    "mxfp8 swiglu 7168 2048 256 8 4096 16384 : 3 1 2048 0 0 0 7\n",  # one too many
    "fp16 swiglu 7168 2048 256 8 4096 16384 : 3 1 2048 0 0 0\n",     # unknown dtype
    "mxfp8 gelu 7168 2048 256 8 4096 16384 : 3 1 2048 0 0 0\n",      # unknown activation
    "mxfp8 swiglu 7168 2048 256 8 4096 1e5 : 3 1 2048 0 0 0\n",      # not an integer
    "mxfp8 swiglu 7168 2048 256 8 4096 16384 : 4 1 2048 0 0 0\n",    # gemm out of range
    "mxfp8 swiglu 7168 2048 256 8 4096 16384 : 3 2 2048 0 0 0\n",    # down_fp8 not 0/1
    "mxfp8 swiglu 7168 2048 256 8 4096 16384 : 3 1 -1 0 0 0\n",      # negative band
    "mxfp8 swiglu 7168 2048 256 8 4096 16384 : 3 1 2048 2 0 0\n",    # fc2_reduce not 0/1
    "mxfp8 swiglu 7168 2048 256 8 4096 16384 : 3 1 2048 0 17 0\n",   # blocks_per_cu out of range
    "mxfp8 swiglu 7168 2048 256 8 4096 16384 : 3 1 2048 0 0 4\n",    # load_balance out of range
    "mxfp8 swiglu 7168 2048 256 8 4096 16384 : 3 1 99999999999 0 0 0\n",  # beyond 32 bits
    # a malformed line after a line of another shape is still an error
    "bf16 swiglu 64 128 8 2 1 10 : 0 1 0 0 0 0\nmxfp8 swiglu 7168 2048 256 8 4096 16384 : 3 1 2048 0 0\n",
])
def test_malformed_lines_are_errors(tmp_path, bad):
    path = _write(tmp_path, bad)
    h = lib.load()
    kn, found = lib.moe_knobs(9, 9, 9, 9, 9, 9), ctypes.c_int32(7)
    st = h.moe_knob_cache_lookup(os.fsencode(path), ctypes.byref(_shape()), 8192, ctypes.byref(kn),
                                 ctypes.byref(found))
    assert st == INVALID and found.value == 0
    assert kn.as_dict() == lib.moe_default_knobs().as_dict()


def test_lookup_null_arguments():
    h = lib.load()
    kn, found = lib.moe_knobs(), ctypes.c_int32(0)
    s = _shape()
    assert h.moe_knob_cache_lookup(None, ctypes.byref(s), 1, ctypes.byref(kn), ctypes.byref(found)) == INVALID
    assert h.moe_knob_cache_lookup(b"/x", None, 1, ctypes.byref(kn), ctypes.byref(found)) == INVALID
    assert h.moe_knob_cache_lookup(b"/x", ctypes.byref(s), 1, None, ctypes.byref(found)) == INVALID
    assert h.moe_knob_cache_lookup(b"/x", ctypes.byref(s), 1, ctypes.byref(kn), None) == INVALID


@pytest.mark.parametrize("knobs,status", [
    ((-1, 1, 0, 0), INVALID), ((4, 1, 0, 0), INVALID), ((0, 2, 0, 0), INVALID), ((0, -1, 0, 0), INVALID),
    ((0, 1, -1, 0), INVALID), ((0, 1, (1 << 20) + 1, 0), INVALID), ((0, 1, 0, 2), INVALID),
    ((0, 1, 0, 0, -1), INVALID), ((0, 1, 0, 0, 17), INVALID), ((0, 1, 0, 0, 0, -1), INVALID),
    ((0, 1, 0, 0, 0, 4), INVALID),
])
def test_forward_knobs_rejects_bad_knobs_on_host(knobs, status):
    s = lib.make_shape(256, 512, 8, 2, 16, "bf16")
    h = lib.load()
    P = ctypes.c_void_p
    ws = lib.moe_workspace_bytes(s)
    kn = lib.moe_knobs(*knobs)
    assert h.moe_forward_knobs(ctypes.byref(s), 4, P(FAKE), P(FAKE), P(FAKE), P(FAKE), None, None, P(FAKE), ws,
                               ctypes.byref(kn), None) == status


def test_forward_knobs_host_checks():
    h = lib.load()
    P = ctypes.c_void_p
    s1 = lib.make_shape(256, 512, 8, 1, 16, "bf16")
    ws = lib.moe_workspace_bytes(s1)
    fc2 = lib.moe_knobs(0, 1, 0, 1, 0)
    # the fc2 accumulator lives in the y region: top_k >= 2 only
    assert h.moe_forward_knobs(ctypes.byref(s1), 4, P(FAKE), P(FAKE), P(FAKE), P(FAKE), None, None, P(FAKE), ws,
                               ctypes.byref(fc2), None) == UNSUPPORTED
    # the 16-row decode items' schedule holds at most 65535 m-tiles: forcing
    # them on more than 16 (65535 - E) routed rows is refused
    big = lib.make_shape(128, 128, 256, 8, 1 << 18, "bf16")
    wsb = lib.moe_workspace_bytes(big)
    T_over = 2 * (65535 - 256) + 1  # top-8: 8 T > 16 (65535 - 256)
    assert h.moe_forward_knobs(ctypes.byref(big), T_over, P(FAKE), P(FAKE), P(FAKE), P(FAKE), None, None, P(FAKE),
                               wsb, ctypes.byref(lib.moe_knobs(1, 1, 0, 0, 0)), None) == UNSUPPORTED
    # the prefill-shaped items address activation rows with 31-bit byte offsets
    huge = lib.make_shape(128, 128, 8, 1, 1 << 23, "bf16")
    wsh = lib.moe_workspace_bytes(huge)
    assert h.moe_forward_knobs(ctypes.byref(huge), 1 << 23, P(FAKE), P(FAKE), P(FAKE), P(FAKE), None, None,
                               P(FAKE), wsh, ctypes.byref(lib.moe_knobs(3, 1, 0, 0, 0)), None) == UNSUPPORTED
    s = lib.make_shape(256, 512, 8, 2, 16, "bf16")
    ws = lib.moe_workspace_bytes(s)
    assert h.moe_forward_knobs(ctypes.byref(s), 4, P(FAKE), P(FAKE), P(FAKE), P(FAKE), None, None, P(FAKE), ws - 1,
                               None, None) == WORKSPACE
    assert h.moe_forward_knobs(ctypes.byref(s), 17, P(FAKE), P(FAKE), P(FAKE), P(FAKE), None, None, P(FAKE), ws,
                               None, None) == INVALID
    assert h.moe_forward_knobs(ctypes.byref(s), 0, None, None, None, None, None, None, None, 0, None, None) == OK


def test_shipped_cache_parses():
    """Every line of the package's knob cache is well formed (a lookup of a
    shape no line names must read the whole file without an error)."""
    path = lib.KNOB_CACHE_PATH
    assert os.path.exists(path)
    h = lib.load()
    s = lib.make_shape(128, 128, 1, 1, 1, "bf16")
    kn, found = lib.moe_knobs(), ctypes.c_int32(0)
    assert h.moe_knob_cache_lookup(os.fsencode(path), ctypes.byref(s), 1, ctypes.byref(kn),
                                   ctypes.byref(found)) == OK
    assert found.value == 0
    lines = [ln.split("#")[0].split() for ln in open(path)]
    assert any(lines), "the shipped cache holds at least one entry"


def test_shipped_cache_is_the_recorded_sweep(tmp_path):
    """The package's knob cache is what the sweep tool writes from the
    committed sweep measurements (profiles/knob_sweep.json)."""
    from mixture_experts_layer_sort_amd import tune

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    out = tmp_path / "cache.txt"
    tune.main(["--from-json", os.path.join(root, "profiles", "knob_sweep.json"), "--out", str(out)])

    def body(path):
        return [ln for ln in open(path) if not ln.startswith("# written by")]

    assert body(out) == body(lib.KNOB_CACHE_PATH)
