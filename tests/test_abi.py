"""libattn's C ABI on the CPU: the library loads, exports every function that
include/attn.h declares, and rejects bad arguments with the documented status
before any HIP call. No call here reaches a kernel launch: every call either
fails validation or is a host-only size/plan query."""
import ctypes
import os
import re

import pytest
import torch

import scaled_dot_product_flashattention_amd as sdpa
from scaled_dot_product_flashattention_amd import build as attn_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

OK, E_NULLPTR, E_SHAPE, E_UNSUPPORTED, E_ALIGN, E_WORKSPACE, E_HIP, E_ARG, E_SCRATCH_LIMIT = range(9)
NOALLOC_SCRATCH_BYTES = 64 << 20
BHSD, BSHD = 0, 1
F32, F16, BF16 = 0, 1, 2


N_TILES = {64: 6, 128: 4}  # tile variants of the 16-bit fused kernel per head size


def SPLIT(g):  # heads in groups of g
    return 0x10000 | g


# fake, never dereferenced device addresses (validation fails before any use)
A16 = 0x10000
A16_2 = 0x20000


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(attn_build.library_path()):
        attn_build.build()
    return sdpa.load_library()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(attn_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"attn_fwd", "attn_fwd_splitk", "attn_fwd_naive", "attn_fwd_plan",
            "attn_fwd_workspace_size", "attn_splitk_workspace_size", "attn_naive_scratch_size",
            "attn_status_string", "attn_version"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"libattn.so does not export {n}"


def test_version_and_status_strings(lib):
    assert lib.attn_version() >= 10000
    seen = set()
    for s in range(9):
        txt = sdpa.attn_status_string(s)
        assert txt and txt not in seen
        seen.add(txt)
    assert sdpa.attn_status_string(99) == "unknown status"


def call(lib, fn="attn_fwd", q=A16, k=A16, v=A16, o=A16_2, lse=None, B=1, H=2, Sq=128, Sk=128,
         d=64, scale=0.125, causal=0, layout=BHSD, dtype=BF16, kv_len=None, extra=None):
    args = [q, k, v, o, lse, B, H, Sq, Sk, d, scale, causal, layout, dtype, kv_len]
    if fn == "attn_fwd_splitk":
        args += extra if extra is not None else [4, None, 0]
    elif fn == "attn_fwd_noalloc":
        pass  # no workspace arguments
    else:
        args += extra if extra is not None else [None, 0]
    return getattr(lib, fn)(*args, None)


@pytest.mark.parametrize("fn", ["attn_fwd", "attn_fwd_splitk", "attn_fwd_naive", "attn_fwd_noalloc"])
def test_validation_statuses(lib, fn):
    assert call(lib, fn, q=None) == E_NULLPTR
    assert call(lib, fn, k=None) == E_NULLPTR
    assert call(lib, fn, v=None) == E_NULLPTR
    assert call(lib, fn, o=None) == E_NULLPTR
    for bad in (dict(B=0), dict(H=0), dict(Sq=0), dict(Sk=0), dict(B=-3),
                dict(B=1 << 16, H=1 << 10, Sq=1 << 10)):
        assert call(lib, fn, **bad) == E_SHAPE, bad
    for bad in (dict(d=96), dict(d=256), dict(d=0), dict(layout=2), dict(layout=-1),
                dict(dtype=3), dict(dtype=-1), dict(layout=SPLIT(3)), dict(layout=SPLIT(0)),
                dict(layout=SPLIT(4)), dict(layout=0x20000 | 2)):
        assert call(lib, fn, **bad) == E_UNSUPPORTED, bad
    for bad in (float("nan"), float("inf"), float("-inf"), -0.5):
        assert call(lib, fn, scale=bad) == E_ARG, bad
    assert call(lib, fn, q=A16 + 8) == E_ALIGN
    assert call(lib, fn, o=A16_2 + 2) == E_ALIGN
    assert call(lib, fn, lse=A16 + 2) == E_ALIGN
    assert call(lib, fn, kv_len=A16 + 1) == E_ALIGN


def test_workspace_statuses(lib):
    # decode shape: the plan splits, so attn_fwd needs a workspace
    shape = dict(B=8, H=32, Sq=1, Sk=32768, d=128)
    n = ctypes.c_int(0)
    assert lib.attn_fwd_plan(8, 32, 1, 32768, 128, BF16, 0, ctypes.byref(n)) == OK
    assert n.value > 1
    need = lib.attn_fwd_workspace_size(8, 32, 1, 32768, 128, BF16, 0)
    assert need == 8 * 32 * 1 * n.value * (128 + 4) * 4
    assert call(lib, **shape, extra=[None, 0]) == E_WORKSPACE
    assert call(lib, **shape, extra=[A16, need - 1]) == E_WORKSPACE
    assert call(lib, **shape, extra=[A16 + 4, need]) == E_ALIGN
    # explicit split count
    assert call(lib, "attn_fwd_splitk", extra=[0, A16, 1 << 30]) == E_SHAPE
    assert call(lib, "attn_fwd_splitk", extra=[4, None, 0]) == E_WORKSPACE
    need4 = lib.attn_splitk_workspace_size(1, 2, 128, 64, 4)
    assert need4 == 1 * 2 * 128 * 4 * (64 + 4) * 4
    assert call(lib, "attn_fwd_splitk", extra=[4, A16, need4 - 4]) == E_WORKSPACE
    # naive scratch: fp32 S plus P in the input type, rows padded to 64 keys
    need_n = lib.attn_naive_scratch_size(1, 2, 128, 100, BF16)
    assert need_n == 1 * 2 * 128 * 128 * (4 + 2)
    assert lib.attn_naive_scratch_size(1, 2, 128, 100, F32) == 1 * 2 * 128 * 128 * 8
    assert call(lib, "attn_fwd_naive", Sk=100, extra=[None, 0]) == E_WORKSPACE
    assert call(lib, "attn_fwd_naive", Sk=100, extra=[A16, need_n - 1]) == E_WORKSPACE
    assert call(lib, "attn_fwd_naive", Sk=100, extra=[A16 + 8, need_n]) == E_ALIGN


def test_noalloc_scratch_limit(lib):
    """attn_fwd_noalloc refuses, before any HIP call, a plan whose workspace
    exceeds its static buffer; the size query says how much it would need."""
    shape = (1024, 32, 1, 32768, 128)
    need = lib.attn_fwd_workspace_size(*shape, BF16, 0)
    assert need > NOALLOC_SCRATCH_BYTES
    B, H, Sq, Sk, d = shape
    assert call(lib, "attn_fwd_noalloc", B=B, H=H, Sq=Sq, Sk=Sk, d=d) == E_SCRATCH_LIMIT
    assert "ATTN_NOALLOC_SCRATCH_BYTES" in sdpa.attn_status_string(E_SCRATCH_LIMIT)
    # the largest decode shape of the study fits
    assert lib.attn_fwd_workspace_size(8, 32, 1, 32768, 128, BF16, 0) <= NOALLOC_SCRATCH_BYTES
    # and the header states the limit the library uses
    text = open(HEADER).read()
    assert "#define ATTN_NOALLOC_SCRATCH_BYTES (64u << 20)" in text


def test_plan_and_size_queries(lib):
    n = ctypes.c_int(-1)
    # prefill shapes never split and need no workspace
    for shp in ((1, 16, 4096, 4096, 64), (2, 16, 8192, 8192, 128), (32, 12, 512, 512, 64),
                (1, 2, 256, 256, 64)):
        assert lib.attn_fwd_plan(*shp, BF16, 0, ctypes.byref(n)) == OK and n.value == 1
        assert lib.attn_fwd_workspace_size(*shp, BF16, 0) == 0
    # single query over many keys splits; few keys do not
    assert lib.attn_fwd_plan(8, 32, 1, 32768, 128, BF16, 0, ctypes.byref(n)) == OK and n.value == 8
    assert lib.attn_fwd_plan(1, 1, 1, 100, 64, BF16, 0, ctypes.byref(n)) == OK and n.value == 1
    # few (batch, head, 128-query tile) workgroups over long keys, 16-bit: the
    # fused kernel over key ranges, about 512 workgroups in all, at least
    # 1024 keys per range, at most 64 ranges
    for shp, want in (((1, 32, 64, 32768, 128), 16), ((2, 32, 128, 16384, 64), 8),
                      ((1, 16, 128, 65536, 64), 32), ((1, 1, 2, 131072, 64), 64),
                      ((1, 64, 128, 4096, 128), 4), ((1, 128, 128, 4096, 64), 4),
                      ((1, 64, 200, 8192, 64), 4), ((1, 1, 7, 5000, 64), 4)):
        for dt in (BF16, F16):
            assert lib.attn_fwd_plan(*shp, dt, 0, ctypes.byref(n)) == OK and n.value == want, shp
        B, H, Sq, Sk, d = shp
        assert lib.attn_fwd_workspace_size(*shp, BF16, 0) == B * H * Sq * want * (d + 4) * 4
        # fp32 never splits a prefill shape
        assert lib.attn_fwd_plan(*shp, F32, 0, ctypes.byref(n)) == OK and n.value == 1
        assert lib.attn_fwd_workspace_size(*shp, F32, 0) == 0
    # ... and not when the workgroups fill the compute units or the rows see
    # fewer than 4096 keys
    for shp in ((1, 256, 128, 8192, 64), (1, 128, 128, 2048, 128), (1, 4, 2000, 4000, 64)):
        assert lib.attn_fwd_plan(*shp, BF16, 0, ctypes.byref(n)) == OK and n.value == 1, shp
    # causal rows see at most Sq keys
    assert lib.attn_fwd_plan(1, 8, 2048, 8192, 128, BF16, 0, ctypes.byref(n)) == OK and n.value == 4
    assert lib.attn_fwd_plan(1, 8, 2048, 8192, 128, BF16, 1, ctypes.byref(n)) == OK and n.value == 1
    assert lib.attn_fwd_workspace_size(1, 8, 2048, 8192, 128, BF16, 1) == 0
    assert lib.attn_fwd_plan(1, 2, 8192, 8192, 64, BF16, 1, ctypes.byref(n)) == OK and n.value == 4
    assert lib.attn_fwd_plan(8, 32, 1, 32768, 128, BF16, 1, ctypes.byref(n)) == OK and n.value == 1
    # the fused kernel over key ranges runs one fixed variant
    t = ctypes.c_int(-1)
    assert lib.attn_fwd_tile_choice(1, 32, 64, 32768, 128, BF16, 0, ctypes.byref(t)) == OK and t.value == 1
    assert lib.attn_fwd_tile_choice(2, 32, 128, 16384, 64, F16, 0, ctypes.byref(t)) == OK and t.value == 1
    # rejected arguments
    assert lib.attn_fwd_plan(0, 1, 1, 1, 64, BF16, 0, ctypes.byref(n)) == E_SHAPE
    assert lib.attn_fwd_plan(1, 1, 1, 1, 80, BF16, 0, ctypes.byref(n)) == E_UNSUPPORTED
    assert lib.attn_fwd_plan(1, 1, 1, 1, 64, 7, 0, ctypes.byref(n)) == E_UNSUPPORTED
    assert lib.attn_fwd_plan(1, 1, 1, 1, 64, BF16, 0, None) == E_NULLPTR
    assert lib.attn_fwd_workspace_size(0, 1, 1, 1, 64, BF16, 0) == 0
    assert lib.attn_splitk_workspace_size(1, 1, 1, 64, 0) == 0
    assert lib.attn_naive_scratch_size(1, 1, 1, 1, 9) == 0


def qkv(lib, x=A16, w=A16, q=A16_2, k=A16_2, v=A16_2, B=1, S=128, D=256, H=2, d=64,
        layout=BHSD, dtype=BF16):
    return lib.attn_qkv_proj(x, w, q, k, v, B, S, D, H, d, layout, dtype, None)


def test_qkv_proj_validation(lib):
    for bad in (dict(x=None), dict(w=None), dict(q=None), dict(k=None), dict(v=None)):
        assert qkv(lib, **bad) == E_NULLPTR, bad
    for bad in (dict(B=0), dict(S=0), dict(H=0), dict(D=0), dict(D=96), dict(D=32), dict(d=0),
                dict(d=12), dict(B=1 << 16, S=1 << 16)):
        assert qkv(lib, **bad) == E_SHAPE, bad
    for bad in (dict(dtype=F32), dict(dtype=5), dict(layout=2), dict(layout=SPLIT(3))):
        assert qkv(lib, **bad) == E_UNSUPPORTED, bad
    for bad in (dict(x=A16 + 8), dict(w=A16 + 2), dict(q=A16_2 + 4), dict(v=A16_2 + 8)):
        assert qkv(lib, **bad) == E_ALIGN, bad


def smx(lib, x=A16, y=A16_2, lse=None, rows=4, n=64, scale=1.0, dtype=BF16, mode=0):
    return lib.attn_softmax_rows(x, y, lse, rows, n, scale, dtype, mode, None)


def test_softmax_rows_validation(lib):
    assert smx(lib, x=None) == E_NULLPTR and smx(lib, y=None) == E_NULLPTR
    for bad in (dict(rows=0), dict(rows=-1), dict(rows=1 << 31), dict(n=0), dict(n=12),
                dict(n=6, dtype=F32)):
        assert smx(lib, **bad) == E_SHAPE, bad
    for bad in (dict(dtype=3), dict(mode=2), dict(mode=-1)):
        assert smx(lib, **bad) == E_UNSUPPORTED, bad
    for bad in (float("nan"), float("inf"), -1.0):
        assert smx(lib, scale=bad) == E_ARG, bad
    for bad in (dict(x=A16 + 8), dict(y=A16_2 + 4), dict(lse=A16 + 2)):
        assert smx(lib, **bad) == E_ALIGN, bad


def test_python_binding_rejects_host_tensors(lib):
    q = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        sdpa.attn_fwd(q, q, q)
    assert sdpa.attn_fwd_plan(8, 32, 1, 32768, 128, torch.bfloat16) == 8
    assert sdpa.attn_fwd_plan(1, 8, 2048, 8192, 128, torch.bfloat16) == 4
    assert sdpa.attn_fwd_plan(1, 8, 2048, 8192, 128, torch.bfloat16, causal=True) == 1
    assert sdpa.attn_fwd_workspace_size(1, 8, 2048, 8192, 128, torch.bfloat16) == 8 * 2048 * 4 * 132 * 4
    with pytest.raises(sdpa.AttnError) as ei:
        sdpa.attn_fwd_plan(1, 1, 1, 1, 96, torch.bfloat16)
    assert ei.value.status == E_UNSUPPORTED


def test_layout_names():
    """The binding's layout names map to the header's codes and tensor shapes."""
    from scaled_dot_product_flashattention_amd.api import layout_code, layout_shape
    assert layout_code("bhsd") == 0 and layout_code("bshd") == 1
    assert layout_code("split:4") == SPLIT(4)
    assert layout_shape("bhsd", 2, 8, 5, 64) == (2, 8, 5, 64)
    assert layout_shape("bshd", 2, 8, 5, 64) == (2, 5, 8, 64)
    assert layout_shape("split:4", 2, 8, 5, 64) == (2, 2, 5, 4, 64)
    with pytest.raises(ValueError):
        layout_code("bsdh")


def test_tile_queries(lib):
    """Variant counts and descriptions; every variant fits gfx950's 160 KiB
    of LDS and 1024 threads per workgroup."""
    for d in (64, 128):
        assert lib.attn_fwd_tile_count(d, F32) == 1
        for dt in (F16, BF16):
            n = lib.attn_fwd_tile_count(d, dt)
            assert n == N_TILES[d]
            for t in range(n):
                info = sdpa.attn_fwd_tile_info(d, {F16: torch.float16, BF16: torch.bfloat16}[dt], t)
                assert info["rows"] % 128 == 0 and info["keys"] in (32, 64, 128)
                assert info["waves"] in (4, 8) and 0 < info["lds_bytes"] <= 160 * 1024
                assert info["stages"] >= 2
    assert lib.attn_fwd_tile_count(96, BF16) == 0 and lib.attn_fwd_tile_count(64, 5) == 0
    info = sdpa.api.TileInfo()
    assert lib.attn_fwd_tile_info(64, BF16, 0, None) == E_NULLPTR
    assert lib.attn_fwd_tile_info(96, BF16, 0, ctypes.byref(info)) == E_UNSUPPORTED
    for bad in ((64, BF16, N_TILES[64]), (64, BF16, -1), (128, F32, 1), (128, BF16, N_TILES[128])):
        assert lib.attn_fwd_tile_info(*bad, ctypes.byref(info)) == E_ARG, bad


def test_tile_choice_covers_every_shape(lib):
    """The compiled table gives a valid variant for every shape, including
    the extremes of both grid axes (clamped), and fp32 has one variant."""
    t = ctypes.c_int(-5)
    for d in (64, 128):
        for causal in (0, 1):
            for B, H, Sq, Sk in ((1, 1, 1, 1), (1, 1, 1, 1 << 30), (1, 16, 4096, 4096),
                                 (1 << 14, 1 << 15, 2, 3), (1, 1, 1 << 30, 7), (7, 3, 333, 5000)):
                assert lib.attn_fwd_tile_choice(B, H, Sq, Sk, d, BF16, causal, ctypes.byref(t)) == OK
                assert 0 <= t.value < N_TILES[d], (d, causal, B, H, Sq, Sk, t.value)
                assert lib.attn_fwd_tile_choice(B, H, Sq, Sk, d, F32, causal, ctypes.byref(t)) == OK
                assert t.value == 0
    assert lib.attn_fwd_tile_choice(1, 1, 1, 1, 64, BF16, 0, None) == E_NULLPTR
    assert lib.attn_fwd_tile_choice(0, 1, 1, 1, 64, BF16, 0, ctypes.byref(t)) == E_SHAPE


def test_qkv_proj_tiling_choice(lib):
    """The projection's tiling from the round counts on 256 CUs: 128 x 192
    tiles (two per CU) unless 256 x 256 tiles need clearly fewer rounds."""
    t = ctypes.c_int(-5)
    cases = [  # (B, S, H, d, tiling): medium and BERT tokens stay on the first
        (1, 4096, 16, 64, 0),    # 512 tiles, one round either way
        (32, 512, 12, 64, 0),    # 1536 tiles: three rounds either way
        (1, 16384, 32, 64, 1),   # 4096 tiles: eight rounds against six
        (1, 4096, 20, 64, 1),    # 640 tiles: two rounds against one
        (1, 1, 1, 8, 0),
    ]
    for B, S, H, d, want in cases:
        assert lib.attn_qkv_proj_tiling(B, S, H, d, 256, ctypes.byref(t)) == OK
        assert t.value == want, (B, S, H, d, t.value)
    # with fewer CUs the large-product tiling comes sooner, never for one round
    assert lib.attn_qkv_proj_tiling(1, 4096, 16, 64, 64, ctypes.byref(t)) == OK and t.value in (0, 1)
    assert lib.attn_qkv_proj_tiling(1, 4096, 16, 64, 256, None) == E_NULLPTR
    for bad in ((0, 1, 1, 8, 256), (1, 0, 1, 8, 256), (1, 1, 0, 8, 256), (1, 1, 1, 0, 256), (1, 1, 1, 8, 0)):
        assert lib.attn_qkv_proj_tiling(*bad, ctypes.byref(t)) == E_SHAPE, bad


def test_tile_table_entries():
    """Every entry of the committed table names an existing variant."""
    path = os.path.join(ROOT, "scaled_dot_product_flashattention_amd", "csrc", "tile_table.inc")
    text = open(path).read()
    body = text[text.index("kTileTable"):]
    rows = re.findall(r"\{([0-9, ]+)\},", body)
    consts = dict(re.findall(r"constexpr int (\w+) = (\d+);", text))
    nr = int(consts["kTuneRowsBuckets"])
    assert len(rows) == 2 * 2 * nr
    for i, r in enumerate(rows):
        vals = [int(x) for x in r.split(",")]
        assert len(vals) == int(consts["kTuneKeysBuckets"])
        d = 64 if i < 2 * nr else 128  # [head size][masking][rows]
        assert all(0 <= x < N_TILES[d] for x in vals)


def tiled(lib, tile=0, q=A16, k=A16, v=A16, o=A16_2, dtype=BF16, d=64, scale=0.125, n_split=1,
          ws=None, ws_bytes=0, B=1, H=2, Sq=8, Sk=8):
    return lib.attn_fwd_tiled(q, k, v, o, None, B, H, Sq, Sk, d, scale, 0, BHSD, dtype, None, tile,
                              n_split, ws, ws_bytes, None)


def test_tiled_validation(lib):
    for bad in (-2, N_TILES[64], 100):
        assert tiled(lib, tile=bad) == E_ARG, bad
    assert tiled(lib, tile=1, dtype=F32) == E_ARG
    assert tiled(lib, q=None) == E_NULLPTR
    assert tiled(lib, d=96) == E_UNSUPPORTED
    assert tiled(lib, o=A16 + 8) == E_ALIGN
    assert tiled(lib, scale=-1.0) == E_ARG
    # key splits: n_split >= 1, 16-bit types only, a workspace of the
    # split-K size (rows * n_split * (d + 4) floats), 16-byte aligned
    need = lib.attn_splitk_workspace_size(1, 2, 8, 64, 4)
    assert need == 2 * 8 * 4 * 68 * 4
    assert tiled(lib, n_split=0) == E_ARG
    assert tiled(lib, n_split=-3) == E_ARG
    assert tiled(lib, n_split=4, dtype=F32, ws=A16, ws_bytes=need) == E_UNSUPPORTED
    assert tiled(lib, n_split=4) == E_WORKSPACE
    assert tiled(lib, n_split=4, ws=A16, ws_bytes=need - 1) == E_WORKSPACE
    assert tiled(lib, n_split=4, ws=A16 + 8, ws_bytes=need) == E_ALIGN
    # record indices past int32, and key-range ends past int32
    assert tiled(lib, n_split=1 << 20, B=1, H=64, Sq=64, ws=A16, ws_bytes=1 << 62) == E_SHAPE
    assert tiled(lib, n_split=1 << 20, Sq=2, Sk=(1 << 31) - 64, H=1, ws=A16, ws_bytes=1 << 62) == E_SHAPE


def test_binding_buffer_checks():
    """Caller-supplied buffers must sit on the inputs' device, be dense and
    have the stated shape and dtype (host-only check, before any launch)."""
    from scaled_dot_product_flashattention_amd.api import _check_buffer
    cpu, gpu = torch.device("cpu"), torch.device("cuda:0")
    good = torch.zeros(2, 3, 4, dtype=torch.float32)
    _check_buffer("lse", good, cpu, (2, 3, 4), torch.float32)
    for args in ((good, gpu, (2, 3, 4), torch.float32),          # wrong device
                 (good, cpu, (2, 3, 5), torch.float32),          # wrong shape
                 (good, cpu, (2, 3, 4), torch.bfloat16),         # wrong dtype
                 (good.transpose(0, 2), cpu, None, None),        # not dense
                 (None, cpu, None, None)):                        # not a tensor
        with pytest.raises(ValueError):
            _check_buffer("x", *args)


def test_header_is_c(tmp_path):
    """include/attn.h is plain C: a C99 translation unit that includes it and
    takes the address of every declared function compiles without warnings."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    names = declared_functions()
    src = tmp_path / "use_attn.c"
    src.write_text('#include "attn.h"\n#include <stddef.h>\ntypedef void (*any_fn)(void);\n'
                   'int main(void) {\n'
                   + "".join(f"    any_fn p_{n} = (any_fn)&{n}; (void)p_{n};\n" for n in names)
                   + "    return ATTN_OK + ATTN_LAYOUT_SPLIT(2) * 0;\n}\n")
    res = subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", f"-I{ROOT}/include",
                          "-c", str(src), "-o", str(tmp_path / "use_attn.o")],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
