"""CPU checks of the C ABI: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host (no GPU involved:
every call here returns before anything is launched)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lp.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\*?\s+\*?(lp_[a-z_0-9]+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    from entropy_chunked_row_amd import _lib
    return _lib.load()


def test_header_lists_the_entry_points():
    names = header_functions()
    for want in ("lp_logprobs_entropy", "lp_lm_head_logprobs_entropy", "lp_lm_head_logprobs_entropy_backward",
                 "lp_lm_head_workspace_bytes", "lp_kl_full_vocab", "lp_prob_diff", "lp_version",
                 "lp_status_string", "lp_last_error"):
        assert want in names


def test_every_declared_symbol_is_exported(lib):
    from entropy_chunked_row_amd import _lib
    for name in header_functions():
        assert hasattr(lib, name), name
        assert name in _lib.SIGNATURES, f"{name} has no ctypes signature"


def test_probe_library_exports_its_declaration():
    """The bench-only read probe (include/lp_probe.h) is a library of its own;
    it rejects bad arguments before launching anything."""
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "lp_probe.h")).read(), flags=re.S)
    names = re.findall(r"^\s*int\s+(lp_probe_[a-z_0-9]+)\s*\(", text, flags=re.M)
    assert names == ["lp_probe_read", "lp_probe_mfma", "lp_probe_exp", "lp_probe_clock_rates"]
    path = os.path.join(ROOT, "entropy_chunked_row_amd", "liblp_probe.so")
    if not os.path.exists(path):
        pytest.skip("liblp_probe.so not built")
    probe = ctypes.CDLL(path)
    f = probe.lp_probe_read
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    assert f(None, 1024, 64, FAKE, None) == 1
    assert f(FAKE, 1000, 64, FAKE, None) == 1      # not a multiple of 16
    assert f(FAKE, 1024, 0, FAKE, None) == 1
    assert f(FAKE + 8, 1024, 64, FAKE, None) == 1  # misaligned
    for n in names:
        assert hasattr(probe, n), n
    g = probe.lp_probe_mfma
    g.restype = ctypes.c_int
    g.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    assert g(0, 10, FAKE, FAKE, None) == 1
    assert g(256, 0, FAKE, FAKE, None) == 1
    assert g(256, 10, None, FAKE, None) == 1
    assert g(256, 10, FAKE + 4, FAKE, None) == 1  # clocks not 8-byte aligned
    e = probe.lp_probe_exp
    e.restype = ctypes.c_int
    e.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    assert e(0, 10, FAKE, FAKE, None) == 1
    assert e(256, 0, FAKE, FAKE, None) == 1
    assert e(256, 10, FAKE, None, None) == 1
    assert e(256, 10, FAKE, FAKE + 2, None) == 1  # sink not 4-byte aligned
    assert "lp_probe" not in " ".join(header_functions())


def test_version_and_status_strings(lib):
    assert lib.lp_version() >= 100
    assert lib.lp_status_string(0) == b"LP_OK"
    assert lib.lp_status_string(3) == b"LP_ERR_WORKSPACE_TOO_SMALL"
    assert lib.lp_status_string(99) == b"unknown status"


FAKE = 0x10000  # never dereferenced: every call below fails validation first


@pytest.mark.parametrize("args,code", [
    (dict(dtype=7), 1),
    (dict(T=-1), 1),
    (dict(V=0), 1),
    (dict(ld=10), 1),             # ld < V
    (dict(temperature=float("inf")), 1),
    (dict(temperature=float("nan")), 1),
    (dict(logits=None), 1),
    (dict(targets=None), 1),
    (dict(logprob=None), 1),
])
def test_logprobs_entropy_validation(lib, args, code):
    a = dict(logits=FAKE, dtype=0, T=4, V=16, ld=16, targets=FAKE, mask=None, temperature=0.7, chunk=2,
             logprob=FAKE, entropy=FAKE)
    a.update(args)
    st = lib.lp_logprobs_entropy(a["logits"], a["dtype"], a["T"], a["V"], a["ld"], a["targets"], a["mask"],
                                 a["temperature"], a["chunk"], a["logprob"], a["entropy"], None)
    assert st == code
    assert lib.lp_last_error() != b""


def test_empty_input_is_ok_without_launch(lib):
    assert lib.lp_logprobs_entropy(None, 0, 0, 16, 16, None, None, 0.7, 4, None, None, None) == 0
    assert lib.lp_last_error() == b""
    assert lib.lp_kl_full_vocab(None, None, 1, 0, 16, 16, 16, None, None, None, None, None, None, None) == 0
    assert lib.lp_prob_diff(None, None, None, 0, None, None) == 0


def test_workspace_query(lib):
    f = lib.lp_lm_head_workspace_bytes
    assert f(0, 5120, 151936, 4096, 0) > 0
    fw = f(32768, 5120, 151936, 4096, 0)
    bw = f(32768, 5120, 151936, 4096, 1)
    assert fw > 0 and bw > fw
    # forward scratch is O(tile_rows x vocab blocks), far below a [T x V] fp32 buffer
    assert fw < 32768 * 151936 * 4 / 50
    assert f(10, 0, 100, 4, 0) == 0 and f(10, 8, 100, 0, 0) == 0 and f(-1, 8, 100, 4, 0) == 0


@pytest.mark.parametrize("args,code", [
    (dict(tile_rows=0), 1),
    (dict(h=12, ld_h=16, ld_w=16), 2),     # h % 8
    (dict(ld_h=4), 1),
    (dict(temperature=float("nan")), 1),
    (dict(ws_bytes=16), 3),
    (dict(hidden=FAKE + 8), 2),             # not 16-byte aligned
    (dict(targets=None), 1),
])
def test_lm_head_validation(lib, args, code):
    a = dict(hidden=FAKE, ld_h=64, weight=FAKE, ld_w=64, T=8, h=64, V=100, targets=FAKE, mask=None,
             temperature=0.7, tile_rows=4, ws=FAKE, ws_bytes=1 << 30)
    a.update(args)
    st = lib.lp_lm_head_logprobs_entropy(a["hidden"], a["ld_h"], a["weight"], a["ld_w"], a["T"], a["h"], a["V"],
                                         a["targets"], a["mask"], a["temperature"], a["tile_rows"], FAKE, None, None,
                                         a["ws"], a["ws_bytes"], None)
    assert st == code, lib.lp_last_error()


def test_kl_validation(lib):
    assert lib.lp_kl_full_vocab(FAKE, FAKE, 7, 4, 16, 16, 16, FAKE, None, None, None, None, None, None) == 1
    assert lib.lp_kl_full_vocab(FAKE + 2, FAKE, 2, 4, 16, 16, 16, FAKE, None, None, None, None, None, None) == 1
    assert lib.lp_kl_full_vocab(FAKE, FAKE, 1, 4, 16, 8, 16, FAKE, None, None, None, None, None, None) == 1
    # target outputs without targets
    assert lib.lp_kl_full_vocab(FAKE, FAKE, 1, 4, 16, 16, 16, FAKE, None, None, FAKE, None, None, None) == 1
    assert lib.lp_prob_diff(FAKE, FAKE, None, -1, FAKE, None) == 1


@pytest.mark.parametrize("args,code", [
    (dict(T=-1), 1),
    (dict(V=0), 1),
    (dict(tile_rows=0), 1),
    (dict(h_t=0), 1),
    (dict(h_s=12, ld_hs=16, ld_ws=16), 2),   # student h % 8
    (dict(ld_ht=8), 1),                       # teacher ld_h < h
    (dict(ht=FAKE + 8), 2),                   # teacher hidden not 16-byte aligned
    (dict(ws=None), 3),
    (dict(ws_bytes=64), 3),
    (dict(kl=None), 1),
    (dict(targets=None, lps=FAKE), 1),        # target outputs need targets
])
def test_lm_head_kl_validation(lib, args, code):
    a = dict(hs=FAKE, ld_hs=64, ws_=FAKE, ld_ws=64, h_s=64, ht=FAKE, ld_ht=32, wt=FAKE, ld_wt=32, h_t=32, T=8, V=100,
             targets=FAKE, tile_rows=4, kl=FAKE, lps=None, ws=FAKE, ws_bytes=1 << 30)
    a.update(args)
    st = lib.lp_lm_head_kl(a["hs"], a["ld_hs"], a["ws_"], a["ld_ws"], a["h_s"], a["ht"], a["ld_ht"], a["wt"],
                           a["ld_wt"], a["h_t"], a["T"], a["V"], None, a["targets"], None, a["tile_rows"], a["kl"],
                           a["lps"], None, None, None, None, a["ws"], a["ws_bytes"], None)
    assert st == code, lib.lp_last_error()


def test_lm_head_kl_workspace_and_backward_checks(lib):
    f = lib.lp_lm_head_kl_workspace_bytes
    fw, bw = f(16384, 7168, 129280, 4096, 0), f(16384, 7168, 129280, 4096, 1)
    # the forward holds the teacher's fp32 logits of one chunk of min(tile_rows, 4096) rows, never [T x V]
    assert 0 < fw < bw and fw < 4096 * 129536 * 4 * 1.1
    assert f(16384, 7168, 129280, 1024, 0) < 1024 * 129536 * 4 * 1.1
    assert f(16384, 7168, 129280, 64, 0) < 256 * 129536 * 4 * 1.05  # a small tile: one 256-row block
    assert f(65536, 7168, 129280, 65536, 0) < 4096 * 129536 * 4 * 1.5  # the chunk is capped
    # only the 4-byte row index list grows with T
    assert f(65536, 7168, 129280, 4096, 0) - fw <= (65536 - 16384) * 4 + 256
    assert f(8, 0, 100, 4, 0) == 0 and f(8, 64, 100, 0, 1) == 0
    # backward without the forward's saved normalisers
    st = lib.lp_lm_head_kl_backward(FAKE, 64, FAKE, 64, 64, FAKE, 64, FAKE, 64, 64, 8, 100, None, 4, None, FAKE, FAKE,
                                    FAKE, FAKE, FAKE, 1 << 30, None)
    assert st == 1 and b"lse_student" in lib.lp_last_error()
    assert lib.lp_lm_head_kl(None, 64, None, 64, 64, None, 64, None, 64, 64, 0, 100, None, None, None, 4, None,
                             None, None, None, None, None, None, 0, None) == 0


def test_launches_beyond_2_32_work_items_are_refused(lib):
    """Shapes whose launches would exceed 2^32-1 work-items in one dispatch
    are refused on the host (LP_ERR_UNSUPPORTED, nothing launched); the same
    rows with a smaller tile pass the check and only miss the workspace."""
    big = dict(T=1 << 20, V=1 << 30)
    st = lib.lp_lm_head_logprobs_entropy(FAKE, 64, FAKE, 64, big["T"], 64, big["V"], FAKE, None, 1.0, 1 << 20, FAKE,
                                         None, None, FAKE, 1 << 30, None)
    assert st == 2 and b"2^32" in lib.lp_last_error()
    st = lib.lp_lm_head_logprobs_entropy_backward(FAKE, 64, FAKE, 64, big["T"], 64, big["V"], FAKE, None, 1.0,
                                                  1 << 20, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, 1 << 30, None)
    assert st == 2 and b"2^32" in lib.lp_last_error()
    st = lib.lp_lm_head_kl(FAKE, 64, FAKE, 64, 64, FAKE, 64, FAKE, 64, 64, big["T"], 1 << 30, None, None, None,
                           1 << 20, FAKE, None, None, None, None, None, FAKE, 1 << 30, None)
    assert st == 2 and b"2^32" in lib.lp_last_error()
    st = lib.lp_lm_head_logprobs_entropy(FAKE, 64, FAKE, 64, big["T"], 64, 151936, FAKE, None, 1.0, 4096, FAKE,
                                         None, None, FAKE, 1 << 20, None)
    assert st == 3, lib.lp_last_error()  # fits; the 1 MiB workspace is what is short


def test_product_path_has_no_fallback(tmp_path):
    """A missing library is an error, not a silent CPU path."""
    from entropy_chunked_row_amd import _lib
    with pytest.raises(RuntimeError, match="no CPU fallback"):
        _lib._lib_backup = _lib._lib
        _lib._lib = None
        try:
            _lib.load(str(tmp_path / "missing.so"))
        finally:
            _lib._lib = _lib._lib_backup


def test_package_never_imports_the_oracle():
    pkg = os.path.join(ROOT, "entropy_chunked_row_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.replace("Oracle", "").lower() or f.endswith((".hip", ".hpp")) and \
                    "import" not in text, f


def test_misaligned_fp32_arguments_are_rejected(lib):
    """Every fp32 array must be 4-byte aligned: the checks run on the host,
    before any launch, so fake device addresses are enough here."""
    mis = FAKE + 2
    ws = 1 << 30
    # fused forward: a misaligned output
    st = lib.lp_lm_head_logprobs_entropy(FAKE, 64, FAKE, 64, 8, 64, 100, FAKE, None, 1.0, 4, mis, None, None,
                                         FAKE, ws, None)
    assert st == 1 and b"misaligned" in lib.lp_last_error()
    # fused backward: a misaligned gradient output, also with no rows (it would be zero-filled)
    for T in (8, 0):
        st = lib.lp_lm_head_logprobs_entropy_backward(FAKE, 64, FAKE, 64, T, 64, 100, FAKE, None, 1.0, 4, FAKE, FAKE,
                                                      FAKE, None, None, mis, FAKE, ws, None)
        assert st == 1 and b"misaligned" in lib.lp_last_error(), T
    # KL through the heads, forward and backward
    st = lib.lp_lm_head_kl(FAKE, 64, FAKE, 64, 64, FAKE, 64, FAKE, 64, 64, 8, 100, None, None, None, 4, mis, None,
                           None, None, None, None, FAKE, ws, None)
    assert st == 1 and b"misaligned" in lib.lp_last_error()
    st = lib.lp_lm_head_kl_backward(FAKE, 64, FAKE, 64, 64, FAKE, 64, FAKE, 64, 64, 8, 100, None, 4, FAKE, FAKE, mis,
                                    None, None, FAKE, ws, None)
    assert st == 1 and b"misaligned" in lib.lp_last_error()
    # KL on given logits, the prob diff and its aggregates
    assert lib.lp_kl_full_vocab(FAKE, FAKE, 0, 8, 100, 100, 100, mis, None, None, None, None, None, None) == 1
    assert lib.lp_prob_diff(FAKE, mis, None, 8, FAKE, None) == 1
    assert lib.lp_prob_diff_stats(mis, FAKE, None, 8, FAKE, FAKE, ws, None) == 1


def test_fast_tiles_need_32bit_offsets_for_every_operand(lib):
    """The direct-to-LDS tiles form 32-bit per-lane byte offsets for every
    operand; shapes where one would wrap run on the generic tiles (64-bit
    addressing) instead of giving wrong logits or gradients.  Host-only query,
    nothing is launched."""
    f = lib.lp_lm_head_fast_tiles
    # the shipping shapes take the fast tiles, forward and backward
    assert f(32768, 5120, 151936, 5120, 5120, 4096, 0) == 1
    assert f(114688, 5120, 151936, 5120, 5120, 4096, 1) == 1
    assert f(16384, 7168, 129280, 7168, 7168, 4096, 1) == 1
    # h % 64 != 0: generic
    assert f(1024, 520, 4096, 520, 520, 256, 0) == 0
    # any hidden row may be gathered: T x ld_h x 2 bytes past 4 GiB
    assert f(420000, 5120, 151936, 5120, 5120, 4096, 0) == 0
    assert f(419000, 5120, 151936, 5120, 5120, 4096, 0) == 1
    # one 256-row weight block past 4 GiB: a huge ld_w
    assert f(1024, 64, 300, 64, 9 * 2 ** 20, 256, 0) == 0
    assert f(1024, 64, 300, 64, 2 ** 23 - 64, 256, 0) == 1
    # backward: a 256-row block of the dZ buffers over V ~ 9M columns
    assert f(1024, 64, 9_000_000, 64, 64, 256, 0) == 1   # the forward never forms those offsets
    assert f(1024, 64, 9_000_000, 64, 64, 256, 1) == 0
    assert f(1024, 64, 8_000_000, 64, 64, 256, 1) == 1
    # backward: tiles of more than ~8.35M rows (dZ^T rows of pitch tpad)
    assert f(9_000_000, 64, 1000, 64, 64, 9_000_000, 1) == 0
    assert f(9_000_000, 64, 1000, 64, 64, 4096, 1) == 1
    # invalid sizes
    assert f(-1, 64, 100, 64, 64, 4, 0) == -1
    assert f(8, 64, 100, 32, 64, 4, 0) == -1
    assert f(8, 64, 100, 64, 64, 0, 0) == -1


def test_noalloc_forward_checks_before_touching_the_device(lib):
    """The no-alloc forward refuses shapes beyond its static scratch (and bad
    arguments) on the host, before it looks up any device; T = 0 is OK."""
    st = lib.lp_lm_head_logprobs_entropy_noalloc(FAKE, 5120, FAKE, 5120, 32768, 5120, 151936, FAKE, None, 0.7, 4096,
                                                 FAKE, None, None, None)
    assert st == 3 and b"static scratch" in lib.lp_last_error()
    # the same rows in 512-row tiles fit the 64 MiB scratch: the workspace form's size query agrees
    assert lib.lp_lm_head_workspace_bytes(32768, 5120, 151936, 512, 0) <= 64 << 20
    assert lib.lp_lm_head_workspace_bytes(32768, 5120, 151936, 4096, 0) > 64 << 20
    assert lib.lp_lm_head_logprobs_entropy_noalloc(FAKE, 64, FAKE, 64, 8, 64, 100, FAKE, None, 0.7, 0, FAKE, None,
                                                   None, None) == 1
    assert lib.lp_lm_head_logprobs_entropy_noalloc(FAKE, 64, FAKE, 64, 8, 64, 100, FAKE, None, 0.7, 4, FAKE + 2,
                                                   None, None, None) == 1
    assert lib.lp_lm_head_logprobs_entropy_noalloc(None, 64, None, 64, 0, 64, 100, None, None, 0.7, 4, None, None,
                                                   None, None) == 0
