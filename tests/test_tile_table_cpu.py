"""Run-time dispatch configuration, no GPU: the GEMV tile table (loaded,
validated as a whole, rejected with a status and the file's line), its
precedence over the built-in table and the heuristic, W4_FORCE_PATH and
W4_LOG."""
import ctypes

import pytest

import bit_weight_only_w4a16_amd as w4

from _util import set_dispatch_env

VP = ctypes.c_void_p
A16 = VP(0x10000)   # aligned, never dereferenced


@pytest.fixture
def L():
    L = w4.lib()
    yield L
    L.w4_tile_table_load(None)


def _table(tmp_path, text, name="t.txt"):
    p = tmp_path / name
    p.write_text(text)
    return str(p)


def test_table_entry_is_used(L, tmp_path):
    base = w4.describe_dispatch(1, 2560, 1536, 32)
    assert "(table)" not in base
    path = _table(tmp_path, "# comment line\n\n"
                            "gemv 2560 1536 32 32 2 2 77 3 0   # trailing comment\n"
                            "gemv 262144 1536 32 16 3 4 0 3 1\n")
    w4.tile_table_load(path)
    assert w4.describe_dispatch(1, 2560, 1536, 32) == \
        "gemv L=32 U=2 W=2 grid=77 stages=3 (table)"
    # grid 0: derived (16 waves per CU for the contiguous kernel)
    assert w4.describe_dispatch(1, 262144, 1536, 32) == \
        "gemv L=16 U=3 W=4 grid=1024 stages=3 contiguous (table)"
    # shapes not in the table keep their previous choice
    assert w4.describe_dispatch(1, 1536, 2048, 32) == w4.describe_dispatch(1, 1536, 2048, 32)
    assert "(table)" not in w4.describe_dispatch(1, 1536, 2048, 32)
    # small M is not a GEMV entry
    assert "(table)" not in w4.describe_dispatch(4, 2560, 1536, 32)
    w4.tile_table_load(None)
    assert w4.describe_dispatch(1, 2560, 1536, 32) == base


def test_generic_entry(L, tmp_path):
    w4.tile_table_load(_table(tmp_path, "gemv 100 1024 256 64 0 1 5 2 0\n"))
    assert w4.describe_dispatch(1, 100, 1024, 256) == \
        "gemv_generic L=64 U=0 W=1 grid=5 stages=2 (table)"


BAD = [
    ("gemm 2560 1536 32 16 3 4 0 2 0", -1, "unknown entry"),
    ("gemv 2560 1536 32 16 3 4 0 2", -1, "10 fields"),
    ("gemv 2560 1536 32 16 3 4 0 2 0 9", -1, "10 fields"),
    ("gemv 2560 1536 32 16 3x 4 0 2 0", -1, "not an integer"),
    ("gemv 2560 1536 64 16 3 4 0 2 0", -2, "group"),
    ("gemv 0 1536 32 16 3 4 0 2 0", -2, "N out of range"),
    ("gemv 2560 1500 32 16 3 4 0 2 0", -2, "multiple of group"),
    ("gemv 2560 1536 32 12 3 4 0 2 0", -2, "L must be"),
    ("gemv 2560 1536 32 16 4 4 0 2 0", -2, "ceil(K / 32 / L) = 3"),
    ("gemv 2560 1536 32 16 9 4 0 2 0", -2, "U must be"),
    ("gemv 2560 1536 512 16 3 4 0 2 0", -2, "even number of groups"),
    ("gemv 2560 1536 32 16 3 5 0 2 0", -2, "waves"),
    ("gemv 2560 1536 32 16 3 4 70000 2 0", -2, "grid"),
    ("gemv 2560 1536 32 16 3 4 -1 2 0", -2, "grid"),
    ("gemv 2560 1536 32 16 3 4 0 4 0", -2, "stages"),
    ("gemv 2560 8192 32 16 16 4 0 2 0", -2, "U must be"),
    ("gemv 2560 6144 32 32 6 4 0 3 0", -2, "three stages"),
    ("gemv 2560 1536 32 16 0 4 0 3 0", -2, "three stages"),
    ("gemv 2560 1536 32 16 3 4 0 2 2", -2, "contig must be"),
    ("gemv 2560 2048 32 16 4 4 0 2 1", -2, "contig needs"),
    ("gemv 2560 1536 32 16 3 2 0 2 1", -2, "contig needs"),
    ("gemv 256 512 32 8 2 4 0 2 1", -2, "contig needs"),
    ("gemv 2560 1536 32 16 3 4 0 2 0\ngemv 2560 1536 32 64 1 4 0 2 0", -1, "listed twice"),
]


@pytest.mark.parametrize("text,status,why", BAD)
def test_malformed_table_is_rejected(L, tmp_path, text, status, why):
    good = _table(tmp_path, "gemv 2560 1536 32 32 2 2 77 3 0\n", "good.txt")
    w4.tile_table_load(good)
    path = _table(tmp_path, "# header\n" + text + "\n")
    st = L.w4_tile_table_load(path.encode())
    assert st == status
    msg = w4.last_error()
    assert why in msg and path in msg
    # the line number of the offending entry (comments count)
    bad_line = 2 if "listed twice" not in why else 3
    assert (":%d:" % bad_line) in msg, msg
    # the previous table stays
    assert "(table)" in w4.describe_dispatch(1, 2560, 1536, 32)


def test_unreadable_table(L, tmp_path):
    assert L.w4_tile_table_load(str(tmp_path / "missing.txt").encode()) == -1
    assert "cannot be read" in w4.last_error()


def test_bad_env_table_fails_every_dispatch(L, tmp_path, monkeypatch):
    path = _table(tmp_path, "gemv 2560 1536 32 16 4 4 0 2 0\n")
    monkeypatch.setenv("W4_TILE_TABLE", path)
    assert L.w4_config_reload() == -2
    assert "W4_TILE_TABLE" in w4.last_error()
    # the calls that dispatch return the table's status before any HIP call
    assert L.w4a16_gemv(A16, 256, 512, 32, A16, A16, 0, VP(0)) == -2
    buf = ctypes.create_string_buffer(64)
    assert L.w4_describe_dispatch(1, 256, 512, 32, buf, 64) == -2
    assert L.w4a16_gemm_smallM(A16, 64, 512, 32, 4, A16, 512, A16, 64, 1, VP(0)) == -2
    # argument errors still come first
    assert L.w4a16_gemv(VP(0), 256, 512, 32, A16, A16, 0, VP(0)) == -1
    # a good table in the environment is used
    good = _table(tmp_path, "gemv 256 512 32 32 1 1 3 2 0\n", "good.txt")
    set_dispatch_env(monkeypatch, W4_TILE_TABLE=good)
    assert w4.describe_dispatch(1, 256, 512, 32) == "gemv L=32 U=1 W=1 grid=3 stages=2 (table)"


def test_force_path(L, monkeypatch):
    set_dispatch_env(monkeypatch, W4_FORCE_PATH="gemv_generic")
    assert w4.describe_dispatch(1, 2560, 1536, 32).startswith("gemv_generic")
    assert "forced gemv_generic" in w4.describe_dispatch(1, 2560, 1536, 32)
    set_dispatch_env(monkeypatch, W4_FORCE_PATH="gemv_contig")
    assert "contiguous" in w4.describe_dispatch(1, 262144, 1536, 32)
    set_dispatch_env(monkeypatch, W4_FORCE_PATH="gemv_tiled")
    assert "contiguous" not in w4.describe_dispatch(1, 262144, 1536, 32)
    set_dispatch_env(monkeypatch, W4_FORCE_PATH="smallm_valu,prefill_regs")
    assert w4.describe_dispatch(8, 12288, 1536, 256).startswith("smallm MT=")
    assert w4.describe_dispatch(24, 12288, 1536, 256).startswith("mfma 16x16x32 block")
    assert "dma-ring" not in w4.describe_dispatch(64, 12288, 1536, 256)
    set_dispatch_env(monkeypatch, W4_FORCE_PATH="no_splitk")
    assert w4.describe_dispatch(24, 12288, 1536, 256).startswith("mfma 16x16x32 dma-ring")
    # the decode-ordered sweep's inline decode is a known name (it applies
    # when a sweep handle is created)
    set_dispatch_env(monkeypatch, W4_FORCE_PATH="ordered_inline")
    assert w4.describe_dispatch(1, 2560, 1536, 32).endswith("(built-in table)")
    monkeypatch.setenv("W4_FORCE_PATH", "gemv_fast")
    assert L.w4_config_reload() == -1
    assert "gemv_fast" in w4.last_error()
    set_dispatch_env(monkeypatch, W4_FORCE_PATH="")
    assert "dma-ring" in w4.describe_dispatch(64, 12288, 1536, 256)


def test_log_prints_each_choice_once(L, monkeypatch, capfd):
    # the call passes validation with a fake pointer, logs, and then fails to
    # launch for want of a device: only where there is none
    if L.w4_device_check() != -6:
        pytest.skip("a HIP device is present: the fake-pointer call would launch")
    set_dispatch_env(monkeypatch, W4_LOG="1")
    for _ in range(3):
        assert L.w4a16_gemv(A16, 256, 512, 32, A16, VP(0x7F000000), 0, VP(0)) == -6
    err = capfd.readouterr().err
    line = "w4a16: M=1 N=256 K=512 group=32: " + w4.describe_dispatch(1, 256, 512, 32)
    assert line.endswith("(built-in table)")
    assert err.count(line) == 1, err


def _committed_table():
    import os
    return os.path.join(os.path.dirname(w4.__file__), "tiles_mi355x.txt")


def test_builtin_table_is_the_searched_table(L):
    """Every entry of the committed search output is what the dispatcher
    picks (from the built-in table), and the built-in header is exactly what
    the generator writes from that file."""
    import os
    from bit_weight_only_w4a16_amd import tune
    path = _committed_table()
    n = 0
    for line in open(path):
        f = line.split("#", 1)[0].split()
        if not f:
            continue
        N, K, g, Lr, U, W, grid, st, ct = (int(v) for v in f[1:])
        d = w4.describe_dispatch(1, N, K, g)
        assert d.endswith("(built-in table)"), d
        assert d.startswith("gemv_generic" if U == 0 else "gemv "), d
        assert ("L=%d U=%d W=%d " % (Lr, U, W)) in d and ("stages=%d" % st) in d, d
        assert (" contiguous" in d) == bool(ct), d
        if grid:
            assert ("grid=%d " % grid) in d, d
        n += 1
    assert n >= 5
    hdr = os.path.join(os.path.dirname(w4.__file__), "csrc", "w4_tiles.h")
    assert open(hdr).read() == tune.header(path)


def test_loaded_table_overrides_builtin(L, tmp_path):
    assert w4.describe_dispatch(1, 12288, 1536, 32).endswith("(built-in table)")
    w4.tile_table_load(_table(tmp_path, "gemv 12288 1536 32 32 2 4 0 2 0\n"))
    assert w4.describe_dispatch(1, 12288, 1536, 32) == \
        "gemv L=32 U=2 W=4 grid=512 stages=2 (table)"


def test_tuner_candidates_are_all_accepted(L, tmp_path):
    """Every tile the search tries passes the table's validation."""
    from bit_weight_only_w4a16_amd import tune
    for N, K, g, _ in tune.SHAPES + [(100, 96, 32, "f32"), (7, 8192, 256, "f32")]:
        lines = [tune.entry(N, K, g, c) for c in tune.candidates(N, K, g)]
        for i, line in enumerate(lines):
            p = _table(tmp_path, line + "\n", "c%d.txt" % i)
            assert L.w4_tile_table_load(p.encode()) == 0, (line, w4.last_error())


def test_sweep_poll_limit_is_read(L, monkeypatch):
    """W4_SWEEP_POLL_LIMIT is read with the configuration; it is a test knob
    and a value out of range is ignored (the default applies)."""
    for v in ("0", "5", "junk", "-3"):
        monkeypatch.setenv("W4_SWEEP_POLL_LIMIT", v)
        assert L.w4_config_reload() == 0
