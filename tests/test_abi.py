"""The C-ABI library loads and exports every function declared in include/*.h, and its host-side
argument checks reject bad calls before any GPU work (no GPU needed)."""
import ctypes
import glob
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^\s*[A-Za-z_][\w\s\*]*?\b(moe_\w+)\s*\(", text, flags=re.M):
            names.add(m.group(1))
    return names


def test_library_exports_every_declared_symbol():
    import expert_cache_offload_amd as m
    lib = ctypes.CDLL(m.LIB_PATH)
    declared = _declared_functions()
    assert {"moe_cache_create", "moe_cache_resize", "moe_route_classify", "moe_fill_misses",
            "moe_expert_ffn", "moe_layer_step"} <= declared
    missing = [n for n in sorted(declared) if not hasattr(lib, n)]
    assert not missing, missing


def test_blob_bytes_and_workspace():
    import expert_cache_offload_amd as m
    assert m.moe_blob_bytes(0, 2048, 768) == 9437184
    assert m.moe_blob_bytes(1, 4096, 2048) == 25952256
    assert m.moe_blob_bytes(2, 6144, 2048) == 20054016
    assert m.moe_blob_bytes(3, 2048, 768) == -1
    assert m.moe_blob_bytes(1, 4000, 2048) == -1
    sh = m.make_shape(48, 128, 8, 2048, 768, 0, 0, 1)
    assert m.moe_workspace_bytes(sh, 1843) > 0
    assert m.moe_workspace_bytes(sh, 0) == 0
    bad = m.make_shape(48, 128, 8, 2000, 768, 0, 0, 1)  # hidden not a multiple of 256
    assert m.moe_workspace_bytes(bad, 1843) == 0


def test_create_rejects_bad_arguments_on_host():
    import expert_cache_offload_amd as m
    sh = m.make_shape(2, 16, 2, 256, 128, 0, 0, 1)
    fake = 1 << 20  # never dereferenced: every check below fails before any HIP call
    with pytest.raises(m.MoeError) as e:
        m.moe_cache_create(sh, 1, 8, fake, fake, fake)  # capacity below min(T*k, E) = 2
    assert e.value.status == m.MOE_E_CAPACITY
    with pytest.raises(m.MoeError) as e:
        m.moe_cache_create(sh, 9, 8, fake, fake, fake)  # capacity above max_capacity
    assert e.value.status == m.MOE_E_CAPACITY
    with pytest.raises(m.MoeError) as e:
        m.moe_cache_create(sh, 4, 8, fake + 4, fake, fake)  # misaligned arena
    assert e.value.status == m.MOE_E_INVALID
    bad = m.make_shape(2, 16, 17, 256, 128, 0, 0, 1)  # top_k > 16
    with pytest.raises(m.MoeError) as e:
        m.moe_cache_create(bad, 4, 8, fake, fake, fake)
    assert e.value.status == m.MOE_E_INVALID
    with pytest.raises(m.MoeError):
        m.moe_route_classify(0, 0, fake, 1, fake)  # null handle
    assert m.moe_status_string(m.MOE_E_BUSY) == "a step is in flight"
