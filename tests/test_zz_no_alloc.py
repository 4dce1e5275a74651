"""moe_grouped_ffn_noalloc (no device allocation: the SwiGLU intermediate lives in
the library's fixed scratch array) against moe_grouped_ffn with a caller
workspace, through the C ABI: two calls in a row, the second on a smaller input,
each bit for bit equal to the workspace call; a shape whose intermediate does not
fit the array is refused before any device work."""
import numpy as np
import pytest
import torch

import synth
from helpers import dev, log, to_dev
from routed_expert_ffn_layer_amd import layer as L
from routed_expert_ffn_layer_amd import moe

pytestmark = pytest.mark.gpu


def _layer_inputs(dtype, T, H, I, E, k, seed, shared):
    I_sh = 128 if shared else 0
    lay = synth.small_layer(dtype, T, H, I, E, k, seed=seed, shared=shared, I_shared=I_sh)
    b = L.LayerBuffers(T, E, k, H, I, dtype, I_shared=I_sh)
    pool = to_dev(lay["experts"])
    stride = pool.shape[1]
    sh = to_dev(lay["shared"]) if shared else None
    x = to_dev(lay["x"])
    L.route(b, to_dev(lay["logits"]))
    return b, pool, stride, sh, x, I_sh


def _both(b, pool, stride, sh, x, I_sh):
    slots = L.identity_slots(b.E)
    T, k, E, H, I = b.T, b.k, b.E, b.H, b.I
    n = T * k
    ref_rows = torch.full((n, H), float("nan"), device=dev())
    ref_sh = torch.full((T, H), float("nan"), device=dev()) if sh is not None else None
    moe.moe_grouped_ffn(b.wdt, pool, stride, slots, sh, I_sh, x, b.offsets, b.sorted_rows, T, k, E, H, I,
                        ref_rows, ref_sh, b.workspace)
    rows = torch.full((n, H), float("nan"), device=dev())
    shr = torch.full((T, H), float("nan"), device=dev()) if sh is not None else None
    moe.moe_grouped_ffn_noalloc(b.wdt, pool, stride, slots, sh, I_sh, x, b.offsets, b.sorted_rows, T, k, E, H, I,
                                rows, shr)
    torch.cuda.synchronize()
    return ref_rows, ref_sh, rows, shr


@pytest.mark.parametrize("dtype", [synth.MXFP4, synth.BF16])
def test_noalloc_matches_workspace_call_twice(dtype):
    # first a grouped-GEMM-sized call (>= 32 pairs per expert), then a smaller
    # weight-streaming one: the second must not see anything of the first
    for T, E, k, shared in ((300, 8, 2, True), (5, 16, 4, False)):
        H, I = 512, 256
        log(f"noalloc dtype={dtype} T={T} E={E} k={k} shared={shared} "
            f"kind={moe.moe_grouped_ffn_kind(T, k, E, H, I, 128 if shared else 0, dtype)}")
        b, pool, stride, sh, x, I_sh = _layer_inputs(dtype, T, H, I, E, k, seed=77 + T, shared=shared)
        ref_rows, ref_sh, rows, shr = _both(b, pool, stride, sh, x, I_sh)
        assert not torch.isnan(ref_rows).any()
        assert torch.equal(rows.view(torch.int32), ref_rows.view(torch.int32))
        if sh is not None:
            assert torch.equal(shr.view(torch.int32), ref_sh.view(torch.int32))


def test_noalloc_refuses_oversized_intermediate():
    # (T*k) rows of I bf16 values beyond the 32 MiB array: refused on the host
    T, k, E, H, I = 4096, 6, 256, 4096, 2048
    assert moe.moe_grouped_ffn_workspace(T, k, E, H, I, 0, moe.MOE_MXFP4) > moe.MOE_NOALLOC_SCRATCH_BYTES
    z = torch.zeros(16, dtype=torch.uint8, device=dev())
    with pytest.raises(moe.MoeError) as e:
        moe.moe_grouped_ffn_noalloc(moe.MOE_MXFP4, z, 16, z, None, 0, z, z, z, T, k, E, H, I, z, None)
    assert e.value.status == moe.MOE_ECAPACITY
