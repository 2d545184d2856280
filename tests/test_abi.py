"""The C ABI library loads, exports every symbol its header declares, and its
argument validation returns the documented status codes.  None of these calls
launches anything, so they run without a GPU."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn_mi355x.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:attn_status|size_t|const char\*)\s+(attn_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def ea():
    import exact_attention_bwd_amd as ea
    return ea


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ("attn_fwd", "attn_bwd_preprocess", "attn_bwd", "attn_bwd_workspace_bytes", "attn_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol(ea):
    out = subprocess.run(["nm", "-D", "--defined-only", ea.lib_path], capture_output=True, text=True, check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    missing = [n for n in _declared() if n not in exported]
    assert not missing, missing
    lib = ctypes.CDLL(ea.lib_path)
    for n in _declared():
        assert getattr(lib, n) is not None


def test_library_is_gfx950_code(ea):
    out = subprocess.run(["strings", ea.lib_path], capture_output=True, text=True, check=True).stdout
    assert "gfx950" in out


def _ws_expected(B, H, N, d, causal):
    """Row statistics (two fp32 per row, rows rounded up to 64), one bf16
    128 x 64 dS tile per (head, 64-row query tile i, 128-key tile j) -- when
    causal only j <= i // 2, counted here tile by tile -- and a bf16 image of K
    per 128-key tile; each part rounded up to 256 bytes.  Causal d = 128 adds
    the persistent kernel's control block: 64 ints and one progress int per
    (head, 256-key tile)."""
    up = lambda x: (x + 255) // 256 * 256  # noqa: E731
    tr, tc = -(-N // 64), -(-N // 128)
    tiles = sum(min(tc, i // 2 + 1) if causal else tc for i in range(tr))
    rows = B * H * tr * 64
    ctrl = up((64 + B * H * -(-N // 256)) * 4) if (causal and d == 128) else 0
    return ctrl + 2 * up(rows * 4) + up(B * H * tiles * 128 * 64 * 2) + up(B * H * tc * 128 * d * 2)


def test_workspace_size(ea):
    for B, H, N, d in ((8, 16, 4096, 128), (1, 1, 100, 64), (2, 3, 333, 128), (1, 2, 1, 64)):
        for causal in (False, True):
            assert ea.attn_bwd_workspace_bytes(B, H, N, d, causal) == _ws_expected(B, H, N, d, causal)
        assert ea.attn_bwd_workspace_bytes(B, H, N, d) == max(_ws_expected(B, H, N, d, c) for c in (False, True))
    # the causal lower triangle is about half the tiles at the headline shape
    full, tri = (ea.attn_bwd_workspace_bytes(8, 16, 4096, 128, c) for c in (False, True))
    assert 0.5 < tri / full < 0.55
    assert ea.attn_bwd_workspace_bytes(0, 16, 4096, 128) == 0
    assert ea.attn_bwd_workspace_bytes(1, 1, 128, 96) == 0                  # unsupported d


def test_binding_rejects_host_workspace(ea):
    import torch
    with pytest.raises(ValueError, match="workspace"):
        ea._workspace(torch.empty(64, dtype=torch.uint8), 16, torch.empty(1))


def _raw(ea):
    return ea._lib


def test_validation_errors_do_not_launch(ea):
    lib = _raw(ea)
    p = ctypes.c_void_p(4096)             # aligned, never dereferenced: validation fails first
    f = ctypes.c_float
    # unsupported head dimension
    assert lib.attn_fwd(p, p, p, p, p, 1, 1, 128, 96, 1, f(0.1), None) == -2
    assert b"head dimension" in lib.attn_last_error()
    # negative size
    assert lib.attn_fwd(p, p, p, p, p, -1, 1, 128, 64, 1, f(0.1), None) == -1
    # non-finite scale
    assert lib.attn_fwd(p, p, p, p, p, 1, 1, 128, 64, 1, f(float("nan")), None) == -1
    assert lib.attn_bwd(p, p, p, p, p, p, p, p, p, p, 1 << 30, 1, 1, 128, 64, 1, f(float("inf")), None) == -1
    # null and misaligned pointers
    assert lib.attn_fwd(None, p, p, p, p, 1, 1, 128, 64, 1, f(0.1), None) == -1
    assert b"q is NULL" in lib.attn_last_error()
    assert lib.attn_fwd(p, ctypes.c_void_p(4098), p, p, p, 1, 1, 128, 64, 1, f(0.1), None) == -1
    assert b"aligned" in lib.attn_last_error()
    assert lib.attn_bwd_preprocess(p, p, ctypes.c_void_p(4097), 1, 1, 128, 64, None) == -1
    # workspace too small
    need = lib.attn_bwd_workspace_bytes(2, 3, 200, 128)
    assert lib.attn_bwd(p, p, p, p, p, p, p, p, p, p, need - 1, 2, 3, 200, 128, 0, f(0.1), None) == -4
    assert b"workspace" in lib.attn_last_error()
    # sizes too large for the grid
    assert lib.attn_fwd(p, p, p, p, p, 1 << 20, 1 << 10, 1 << 20, 64, 0, f(0.1), None) == -2


def test_empty_problems_are_noops(ea):
    lib = _raw(ea)
    f = ctypes.c_float
    # nothing to do: OK without touching any pointer or the GPU
    assert lib.attn_fwd(None, None, None, None, None, 0, 4, 128, 64, 1, f(0.1), None) == 0
    assert lib.attn_fwd(None, None, None, None, None, 2, 4, 0, 128, 0, f(0.1), None) == 0
    assert lib.attn_bwd_preprocess(None, None, None, 2, 0, 64, 64, None) == 0
    assert lib.attn_bwd(None, None, None, None, None, None, None, None, None, None, 0, 0, 1, 1, 64, 1, f(0.1), None) == 0
    assert lib.attn_last_error() == b""


def test_version(ea):
    assert "gfx950" in ea.version()


def test_sparse_validation_errors_do_not_launch(ea):
    lib = _raw(ea)
    p = ctypes.c_void_p(4096)
    f = ctypes.c_float
    # unsupported head dims / head count
    assert lib.attn_sparse_fwd(p, p, p, p, None, p, p, 64, 16, 16, 512, 512, 8, f(0.1), None) == -2
    assert b"576" in lib.attn_last_error()
    assert lib.attn_sparse_fwd(p, p, p, p, None, p, p, 32, 16, 16, 576, 512, 8, f(0.1), None) == -2
    # negative size, non-finite scale
    assert lib.attn_sparse_fwd(p, p, p, p, None, p, p, 64, -1, 16, 576, 512, 8, f(0.1), None) == -1
    assert lib.attn_sparse_fwd(p, p, p, p, None, p, p, 64, 16, 16, 576, 512, 8, f(float("nan")), None) == -1
    # misaligned index list
    assert lib.attn_sparse_fwd(p, p, p, ctypes.c_void_p(4098), None, p, p, 64, 16, 16, 576, 512, 8,
                               f(0.1), None) == -1
    # backward key limit and workspace size
    assert lib.attn_sparse_bwd_workspace_bytes(64, 16, 20000, 576, 512, 8) == 0
    need = lib.attn_sparse_bwd_workspace_bytes(64, 16, 16, 576, 512, 8)
    assert lib.attn_sparse_bwd(p, p, p, p, p, p, p, None, p, p, p, p, need - 1, 64, 16, 16, 576, 512, 8,
                               f(0.1), None) == -4
    assert lib.attn_sparse_bwd(p, p, p, p, p, p, p, None, p, p, p, p, 1 << 40, 64, 16, 20000, 576, 512, 8,
                               f(0.1), None) == -2
    # backward top-k limit: a row's contribution block must stay far below 1 GiB
    assert lib.attn_sparse_bwd_workspace_bytes(64, 16, 16, 576, 512, 65537) == 0
    assert lib.attn_sparse_bwd(p, p, p, p, p, p, p, None, p, p, p, p, 1 << 40, 64, 16, 16, 576, 512, 65537,
                               f(0.1), None) == -2
    assert b"topk" in lib.attn_last_error()


def test_sparse_workspace_size(ea):
    # per-row-block key counts, key offsets, pair list, dS (64 heads per slot,
    # slots padded to 256), the two fp32 scales and the fp16 dK/dV contribution
    # of every slot
    al = lambda x: (x + 255) // 256 * 256  # noqa: E731
    got = ea.attn_sparse_bwd_workspace_bytes(64, 4096, 4096, 512)
    assert got == (al(256 * 4096 * 4) + al(4097 * 4) + al(4096 * 512 * 4) + al(4096 * 512 * 64 * 2)
                   + al(4096 * 512 * 8) + al(4096 * 512 * 1088 * 2))
    assert ea.attn_sparse_bwd_workspace_bytes(128, 300, 280, 100) == (
        al(19 * 280 * 4) + al(281 * 4) + al(300 * 100 * 4) + al(300 * 2 * 256 * 64 * 2)
        + al(300 * 2 * 100 * 8) + al(300 * 2 * 100 * 1088 * 2))
    assert ea.attn_sparse_bwd_workspace_bytes(0, 0, 0, 8) == 0


def test_sparse_empty_is_noop(ea):
    lib = _raw(ea)
    f = ctypes.c_float
    assert lib.attn_sparse_fwd(None, None, None, None, None, None, None, 0, 16, 16, 576, 512, 8, f(0.1), None) == 0
    assert lib.attn_sparse_fwd(None, None, None, None, None, None, None, 64, 0, 16, 576, 512, 8, f(0.1), None) == 0
    assert lib.attn_sparse_bwd(None, None, None, None, None, None, None, None, None, None, None, None, 0,
                               64, 0, 0, 576, 512, 8, f(0.1), None) == 0
