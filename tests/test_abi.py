"""The C-ABI library loads and exports every declared entry point; argument
checks reject bad calls before any device work (runs without a GPU)."""
import ctypes
import os
import re

import pytest

import synth
from routed_expert_ffn_layer_amd import moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "moe.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    L = moe.lib()
    names = _declared()
    assert len(names) >= 20
    for n in names:
        assert hasattr(L, n), n
    assert sorted(moe.EXPORTS) == names


def test_version_and_status_strings():
    L = moe.lib()
    assert moe.moe_abi_version() == 1
    assert L.moe_status_str(0) == b"ok"
    assert L.moe_status_str(moe.MOE_EINVAL) == b"invalid argument"


@pytest.mark.parametrize("wdt,H,I", [(0, 256, 512), (1, 2048, 512), (2, 4096, 2048), (2, 64, 32)])
def test_expert_bytes_matches_layout(wdt, H, I):
    assert moe.moe_expert_bytes(wdt, H, I) == synth.expert_bytes(wdt, H, I)


def test_mxfp4_bytes_of_the_pages_layer_shape():
    assert moe.moe_expert_bytes(moe.MOE_MXFP4, 4096, 2048) == 13369344
    assert moe.moe_expert_bytes(moe.MOE_BF16, 2048, 512) == 6291456


def _rc(fn, *args):
    return fn(*args)


def test_argument_checks_without_device():
    L = moe.lib()
    null = None
    st = None
    assert L.moe_route_topk(null, 4, 0, 2, null, null, st) == moe.MOE_EINVAL       # E = 0
    assert L.moe_route_topk(null, 4, 2048, 2, null, null, st) == moe.MOE_EINVAL    # E > 1024
    assert L.moe_route_topk(null, 4, 8, 9, null, null, st) == moe.MOE_EINVAL      # k > E
    assert L.moe_route_topk(null, -1, 8, 2, null, null, st) == moe.MOE_EINVAL     # T < 0
    assert L.moe_route_topk(null, 4, 8, 2, null, null, st) == moe.MOE_EINVAL      # null logits
    assert L.moe_route_topk(ctypes.c_void_p(8), 4, 8, 2, ctypes.c_void_p(16), ctypes.c_void_p(32), st) == moe.MOE_EINVAL
    assert b"aligned" in L.moe_last_error()
    assert L.moe_route_topk(null, 0, 8, 2, null, null, st) == moe.MOE_OK          # empty batch is a no-op
    assert L.moe_permute(null, 4, 2, 8, null, null, null, null, st) == moe.MOE_EINVAL
    # FFN: bad weight type, misaligned H for bf16, workspace too small
    p = ctypes.c_void_p(1 << 20)
    args = lambda wdt, H, I, ws: (wdt, p, moe.moe_expert_bytes(1, 2048, 512), p, null, 0, p, p, p, 4, 2, 8, H, I, p,
                                  null, p, ws, st)
    assert L.moe_grouped_ffn(*args(7, 2048, 512, 1 << 30)) == moe.MOE_EINVAL
    assert L.moe_grouped_ffn(*args(1, 2000, 512, 1 << 30)) == moe.MOE_EINVAL
    assert L.moe_grouped_ffn(*args(1, 2048, 512, 16)) == moe.MOE_ECAPACITY
    assert L.moe_grouped_ffn_workspace(4, 2, 8, 2048, 512, 0, 1) == 4 * 2 * 512 * 2
    assert L.moe_grouped_ffn_workspace(4, 2, 8, 2048, 512, 256, 0) == (8 + 4) * 512 * 4
    assert L.moe_combine(null, null, null, null, 4, 2, 6, null, 1, st) == moe.MOE_EINVAL   # H % 4
    assert L.moe_combine(p, p, p, null, 4, 2, 8, p, 5, st) == moe.MOE_EINVAL               # bad ydt


def test_cache_create_checks():
    with pytest.raises(moe.MoeError):
        moe.MoeCache(0, 8, 4)
    with pytest.raises(moe.MoeError):
        moe.MoeCache(1, 2000, 4)
    c = moe.MoeCache(2, 8, 4)  # host-only planning handle
    with pytest.raises(moe.MoeError) as e:
        c.lookup_host(0, None, 1)  # wave 1 before wave 0
    assert e.value.status in (moe.MOE_ESTATE, moe.MOE_EINVAL)
    with pytest.raises(moe.MoeError):
        c.lookup_host(5, [1] * 8, 0)  # layer out of range
    c.close()
