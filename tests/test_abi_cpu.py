"""CPU tests of the C ABI: the library loads, exports what include/pa.h
declares, sizes pools as the pages do, and rejects bad arguments before any
GPU work is enqueued (no call here reaches a kernel launch)."""
import ctypes
import os
import re

import pytest

import paged_kv_cache_64_amd as pa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pa.h")

# Fake, aligned, never-dereferenced device addresses for validation paths.
FAKE = 1 << 20


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z_0-9]+)\s*\(", text)))


def _desc(layers=32, blocks=64, bs=16, hkv=8, d=128, dtype=pa.PA_F16):
    return pa.PoolDesc(layers, blocks, bs, hkv, d, dtype)


@pytest.fixture(scope="module")
def lib():
    return pa.load_library()


def test_library_exports_every_declared_symbol(lib):
    declared = _declared()
    assert declared == sorted(pa.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_pool_bytes_matches_the_pages_sizing(lib):
    # one block of one layer, K + V: 16 x 8 x 256 x 2 = 65,536 B
    assert 2 * pa.pa_pool_bytes(_desc(layers=1, blocks=1)) == 65536
    # 32 layers: 2,048 KiB per block
    assert 2 * pa.pa_pool_bytes(_desc(layers=32, blocks=1)) == 2048 * 1024
    # 128 KiB per token over 32 layers
    assert 2 * pa.pa_pool_bytes(_desc(layers=32, blocks=1)) // 16 == 128 * 1024
    assert pa.pa_pool_bytes(_desc(blocks=0)) == 0
    assert lib.pa_pool_bytes(None) == 0


def test_fp8_pool_bytes_halve(lib):
    # an FP8 cache stores one byte per value: 1,024 KiB per block over 32 layers
    fp8 = _desc(layers=32, blocks=1, dtype=pa.PA_FP8_E4M3)
    assert 2 * pa.pa_pool_bytes(fp8) == 1024 * 1024
    assert pa.pa_pool_bytes(_desc(layers=3, blocks=7, dtype=pa.PA_FP8_E4M3)) * 2 == \
        pa.pa_pool_bytes(_desc(layers=3, blocks=7))
    assert pa.pa_pool_bytes(_desc(dtype=3)) == 0


def test_set_scales_validation(lib):
    handle = pa.pa_pool_create(_desc(layers=2, blocks=4, dtype=pa.PA_FP8_E4M3), FAKE, FAKE)
    try:
        pa.pa_pool_set_scales(handle, 1, 0.1, 0.0173)
        for layer, ks, vs in [(-1, 1.0, 1.0), (2, 1.0, 1.0), (0, 0.0, 1.0), (0, 1.0, -1.0),
                              (0, float("nan"), 1.0), (0, 1.0, float("inf")),
                              (0, 1e-45, 1.0)]:       # 1/scale overflows fp32
            assert lib.pa_pool_set_scales(handle, layer, ks, vs) == pa.PA_ERR_INVALID_ARG
        assert lib.pa_pool_set_scales(None, 0, 1.0, 1.0) == pa.PA_ERR_INVALID_ARG
    finally:
        pa.pa_pool_destroy(handle)
    with pytest.raises(ValueError):
        pa.Pool(1, 4, dtype=3, device="cpu")


def test_status_strings(lib):
    for code in (pa.PA_OK, pa.PA_ERR_INVALID_ARG, pa.PA_ERR_UNSUPPORTED, pa.PA_ERR_WORKSPACE,
                 pa.PA_ERR_HIP):
        assert pa.pa_status_string(code)
    assert pa.pa_status_string(42) == "unknown status"


def test_pool_create_checks(lib):
    h = ctypes.c_void_p()
    d = _desc()
    assert lib.pa_pool_create(ctypes.byref(d), FAKE, FAKE, None) == pa.PA_ERR_INVALID_ARG
    assert lib.pa_pool_create(ctypes.byref(d), None, FAKE, ctypes.byref(h)) == pa.PA_ERR_INVALID_ARG
    assert lib.pa_pool_create(ctypes.byref(d), FAKE + 2, FAKE, ctypes.byref(h)) == pa.PA_ERR_INVALID_ARG
    bad = _desc(d=64)
    assert lib.pa_pool_create(ctypes.byref(bad), FAKE, FAKE, ctypes.byref(h)) == pa.PA_ERR_UNSUPPORTED
    bad = _desc(bs=32)
    assert lib.pa_pool_create(ctypes.byref(bad), FAKE, FAKE, ctypes.byref(h)) == pa.PA_ERR_UNSUPPORTED
    handle = pa.pa_pool_create(d, FAKE, FAKE)
    assert handle
    pa.pa_pool_destroy(handle)
    assert lib.pa_pool_destroy(None) == pa.PA_OK


@pytest.fixture
def pool(lib):
    handle = pa.pa_pool_create(_desc(layers=2, blocks=64), FAKE, FAKE)
    yield handle
    pa.pa_pool_destroy(handle)


def test_write_kv_validation(lib, pool):
    assert lib.pa_write_kv(pool, 0, FAKE, FAKE, FAKE, 0, None) == pa.PA_OK       # no-op
    assert lib.pa_write_kv(pool, 2, FAKE, FAKE, FAKE, 4, None) == pa.PA_ERR_INVALID_ARG
    assert lib.pa_write_kv(pool, -1, FAKE, FAKE, FAKE, 4, None) == pa.PA_ERR_INVALID_ARG
    assert lib.pa_write_kv(pool, 0, None, FAKE, FAKE, 4, None) == pa.PA_ERR_INVALID_ARG
    assert lib.pa_write_kv(pool, 0, FAKE, FAKE, FAKE, -1, None) == pa.PA_ERR_INVALID_ARG
    assert lib.pa_write_kv(pool, 0, FAKE + 8, FAKE, FAKE, 4, None) == pa.PA_ERR_INVALID_ARG
    assert lib.pa_write_kv(None, 0, FAKE, FAKE, FAKE, 4, None) == pa.PA_ERR_INVALID_ARG


def _decode(lib, pool, layer=0, q=FAKE, out=FAKE, tables=FAKE, width=16, lens=FAKE, batch=4,
            hq=32, max_ctx=256, scale=0.088, ws=FAKE, ws_bytes=1 << 30):
    return lib.pa_decode(pool, layer, q, out, tables, width, lens, batch, hq, max_ctx, scale, ws,
                         ws_bytes, None)


def test_decode_validation(lib, pool):
    assert _decode(lib, pool, batch=0) == pa.PA_OK                          # no-op
    assert _decode(lib, pool, layer=2) == pa.PA_ERR_INVALID_ARG
    assert _decode(lib, pool, hq=12) == pa.PA_ERR_INVALID_ARG               # not a multiple of 8
    assert _decode(lib, pool, hq=16) == pa.PA_ERR_UNSUPPORTED               # group of 2
    assert _decode(lib, pool, max_ctx=257) == pa.PA_ERR_INVALID_ARG         # > width * 16
    assert _decode(lib, pool, batch=-1) == pa.PA_ERR_INVALID_ARG
    assert _decode(lib, pool, q=None) == pa.PA_ERR_INVALID_ARG
    assert _decode(lib, pool, q=FAKE + 4) == pa.PA_ERR_INVALID_ARG          # misaligned
    assert _decode(lib, pool, scale=float("nan")) == pa.PA_ERR_INVALID_ARG
    assert _decode(lib, pool, batch=70000) == pa.PA_ERR_UNSUPPORTED
    assert _decode(lib, pool, width=(1 << 26) + 1, max_ctx=(1 << 30) + 1) == pa.PA_ERR_UNSUPPORTED  # > 2^30 tokens
    assert pa.pa_decode_workspace_bytes(pool, 4, 32, 256) == 0               # one split: no workspace
    need = pa.pa_decode_workspace_bytes(pool, 4, 32, 4096)
    assert need > 0
    split = dict(width=256, max_ctx=4096)
    assert _decode(lib, pool, ws_bytes=need - 1, **split) == pa.PA_ERR_WORKSPACE
    assert _decode(lib, pool, ws=None, **split) == pa.PA_ERR_WORKSPACE
    assert _decode(lib, pool, ws=FAKE + 16, **split) == pa.PA_ERR_INVALID_ARG   # workspace alignment
    assert lib.pa_decode_merge(pool, FAKE, FAKE, 4, 32, 4096, FAKE, need - 1, None) == pa.PA_ERR_WORKSPACE
    # the appending variant needs both new-token tensors, aligned
    assert lib.pa_append_decode(pool, 0, FAKE, None, FAKE, FAKE, FAKE, 16, FAKE, 4, 32, 256, 0.088,
                                FAKE, 1 << 30, None) == pa.PA_ERR_INVALID_ARG
    assert lib.pa_append_decode(pool, 0, FAKE, FAKE + 8, FAKE, FAKE, FAKE, 16, FAKE, 4, 32, 256,
                                0.088, FAKE, 1 << 30, None) == pa.PA_ERR_INVALID_ARG
    assert lib.pa_decode_partial(pool, 0, FAKE, FAKE, None, FAKE, FAKE, 16, FAKE, 4, 32, 256, 0.088,
                                 FAKE, 1 << 30, None) == pa.PA_ERR_INVALID_ARG


def test_split_plan_and_workspace(lib, pool, monkeypatch):
    monkeypatch.delenv("PA_SPLIT_TOKENS", raising=False)
    for batch, max_ctx in [(1, 256), (8, 4096), (32, 4096), (64, 8192), (256, 8192), (3, 1)]:
        s = pa.pa_decode_split_tokens(pool, batch, 32, max_ctx)
        assert s % 64 == 0 and 256 <= s <= 4096      # at least 4 blocks per wave
        splits = -(-max_ctx // s)
        ws = pa.pa_decode_workspace_bytes(pool, batch, 32, max_ctx)
        if splits == 1:
            assert ws == 0
        else:
            rows = batch * 32 * splits
            assert ws >= rows * (128 + 2) * 4
    assert pa.pa_decode_split_tokens(pool, 1, 32, 256) == 256     # one split, no merge
    assert pa.pa_decode_split_tokens(pool, 8, 32, 4096) == 1024
    assert pa.pa_decode_split_tokens(pool, 32, 32, 4096) == 4096
    monkeypatch.setenv("PA_SPLIT_TOKENS", "128")
    assert pa.pa_decode_split_tokens(pool, 32, 32, 4096) == 128
    monkeypatch.setenv("PA_SPLIT_TOKENS", "100")     # not a multiple of 64: ignored
    assert pa.pa_decode_split_tokens(pool, 32, 32, 4096) % 64 == 0
    assert pa.pa_decode_split_tokens(pool, 32, 32, 4096) != 100


def test_a_library_built_from_other_sources_is_refused(tmp_path):
    """load_library checks the source hash the build embeds: a copy of the
    library whose recorded hash differs from the sources is refused, and so is
    a library without one."""
    from paged_kv_cache_64_amd import build

    data = open(pa.LIB_PATH, "rb").read()
    have = build.built_hash(pa.LIB_PATH)
    assert have == build.source_hash()
    stale = tmp_path / "libpa_stale.so"
    stale.write_bytes(data.replace(have.encode(), b"0" * 64))
    with pytest.raises(RuntimeError, match="other sources"):
        build.check_current(str(stale))
    bare = tmp_path / "libpa_bare.so"
    bare.write_bytes(data.replace(b"pa-source-sha256:", b"xx-source-sha256:"))
    with pytest.raises(RuntimeError, match="other sources"):
        build.check_current(str(bare))
    with pytest.raises(RuntimeError, match="missing"):
        build.check_current(str(tmp_path / "nothing.so"))
    # an edited source changes the hash the loader expects
    src = tmp_path / "pa_kernels.hip"
    src.write_bytes(open(build.SOURCES[-1], "rb").read() + b"\n// edit\n")
    assert build.source_hash(build.SOURCES[:-1] + [str(src)]) != have


def test_the_oracle_rebuilds_a_library_made_from_other_sources(tmp_path):
    from oracle import build as obuild

    lib = str(tmp_path / "liboracle.so")
    obuild.build(lib=lib)
    assert obuild.is_current(lib)
    data = open(lib, "rb").read()
    open(lib, "wb").write(data.replace(obuild.source_hash().encode(), b"f" * 64))
    assert not obuild.is_current(lib)
    assert obuild.is_current(obuild.DEFAULT_LIB) or not os.path.exists(obuild.DEFAULT_LIB)


def test_noalloc_decode_validation(lib, pool):
    """pa_decode_noalloc rejects what pa_decode rejects, and a launch shape whose
    partials would not fit its fixed 32 MiB array, before any device work."""
    f = lib.pa_decode_noalloc
    assert f(pool, 0, FAKE, FAKE, FAKE, 16, FAKE, 0, 32, 0, 0.1, None) == pa.PA_OK      # empty batch
    assert f(None, 0, FAKE, FAKE, FAKE, 16, FAKE, 2, 32, 256, 0.1, None) == pa.PA_ERR_INVALID_ARG
    assert f(pool, 0, FAKE, FAKE, FAKE, 16, FAKE, 2, 30, 256, 0.1, None) == pa.PA_ERR_INVALID_ARG
    assert f(pool, 0, FAKE, FAKE, FAKE, 15, FAKE, 2, 32, 256, 0.1, None) == pa.PA_ERR_INVALID_ARG
    # 1000 sequences of up to 2^20 tokens: 256 splits each, 4.3 GB of partials
    assert lib.pa_decode_workspace_bytes(pool, 1000, 32, 1 << 20) > 32 << 20
    assert f(pool, 0, FAKE, FAKE, FAKE, 1 << 16, FAKE, 1000, 32, 1 << 20, 0.1, None) == pa.PA_ERR_WORKSPACE


def test_binding_structs_match_the_header_layout(tmp_path):
    """Every field of pa_pool_desc and pa_plan_info sits at the same offset, and
    each struct has the same size, in include/pa.h (compiled by the host C
    compiler) as in the ctypes mirror the binding marshals."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no host C compiler")
    structs = {"pa_pool_desc": pa.PoolDesc, "pa_plan_info": pa.PlanInfo}
    lines = ["#include <stdio.h>", "#include <stddef.h>", '#include "pa.h"', "int main(void) {"]
    for cname, cls in structs.items():
        lines.append(f'    printf("{cname} size %zu\\n", sizeof({cname}));')
        for field, _ in cls._fields_:
            lines.append(f'    printf("{cname} {field} %zu\\n", offsetof({cname}, {field}));')
    lines += ["    return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.run([cc, "-std=c11", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                    "-I", "/opt/rocm/include", "-o", str(exe), str(src)], check=True)
    got = {}
    for line in subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.splitlines():
        cname, field, value = line.split()
        got[(cname, field)] = int(value)
    for cname, cls in structs.items():
        assert got[(cname, "size")] == ctypes.sizeof(cls), cname
        for field, _ in cls._fields_:
            assert got[(cname, field)] == getattr(cls, field).offset, (cname, field)
