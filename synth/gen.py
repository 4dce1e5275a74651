"""Random draws, stored-format encodings and the expert slot layout.

Formats
-------
* f32   -- IEEE binary32.
* bf16  -- the upper 16 bits of binary32, produced here with round-to-nearest-even.
* MXFP4 -- OCP Microscaling (MX) v1.0 with E2M1 elements and one E8M0 scale per
  block of 32 consecutive elements along a row (the reduction dimension K of the
  matrix).  Element 2i of a row sits in the low nibble of byte i, element 2i+1 in
  the high nibble.  The encoder follows the spec's conversion rule: the block's
  shared exponent is floor(log2(amax)) - 2 (2 is the largest E2M1 exponent) and
  each element is rounded to nearest-even E2M1, saturating at +-6.

Expert slot layout (the layout experts are kept in, host and device: one expert is one contiguous run of
``expert_bytes`` so a cache fill is a single copy)::

    f32   :  W13 [2I][H] then W2 [H][I], row-major, rows K-contiguous;
             W13 rows 0..I-1 gate, I..2I-1 up
    bf16  :  W13 then W2, each in the tiled layout below
    mxfp4 :  W13 codes, W2 codes, W13 scales, W2 scales, tiled

Tiled layout of a matrix with R rows (R % 16 == 0) and K columns: tiles of 16
rows x KS columns (KS = 32 bf16, 128 MXFP4), row-tile major then column step;
inside a tile, 64 fragments of 16 bytes ordered by f = 16*g + row%16 with
g = (k % KS) // (KS/4).  A bf16 fragment is 8 consecutive k; an MXFP4 fragment
is one 32-element block, and its E8M0 scale is byte f of the tile's 64-byte
scale block.  MXFP4 steps past K are zero padding.  For bf16 and MXFP4 the W13
rows are interleaved per tile: stored row 16t+q is gate row 8t+q (q < 8) or up
row 8t+q-8.  W2 is the down projection.
"""
import numpy as np

F32, BF16, MXFP4 = 0, 1, 2
DTYPE_NAMES = {F32: "f32", BF16: "bf16", MXFP4: "mxfp4"}
DTYPE_BY_NAME = {v: k for k, v in DTYPE_NAMES.items()}

# E2M1 magnitudes by 3-bit code, from the OCP MX v1.0 element table.  Used here
# only to *encode* draws; the oracle decodes with its own table.
_E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
# Midpoints between consecutive magnitudes.  A value exactly on midpoint i is a
# tie between codes i and i+1; nearest-even picks the code whose mantissa bit is 0,
# i.e. the even code.
_E2M1_MID = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], dtype=np.float64)


def rng(base_seed: int, *path: int) -> np.random.Generator:
    """Independent, reproducible stream for (base_seed, path...)."""
    ss = np.random.SeedSequence(entropy=int(base_seed), spawn_key=tuple(int(p) for p in path))
    return np.random.Generator(np.random.PCG64(ss))


def bf16_bits(a) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def e2m1_encode(m) -> np.ndarray:
    """Non-negative magnitudes (already divided by the block scale) -> 3-bit codes,
    round to nearest even, saturating at 6."""
    m = np.asarray(m, dtype=np.float64)
    code = np.zeros(m.shape, dtype=np.uint8)
    for i, b in enumerate(_E2M1_MID):
        code += (m > b).astype(np.uint8)
        if i % 2 == 1:  # tie between odd code i and even code i+1 -> round up
            code += (m == b).astype(np.uint8)
    return code


def mx_quantize(w) -> tuple:
    """float matrix [rows][K] (K % 32 == 0) -> (codes uint8 [rows][K/2], scales uint8 [rows][K/32])."""
    w = np.asarray(w, dtype=np.float64)
    rows, K = w.shape
    assert K % 32 == 0
    blk = w.reshape(rows, K // 32, 32)
    amax = np.abs(blk).max(axis=2)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(amax > 0, amax, 1.0))).astype(np.int64) - 2
    e = np.where(amax > 0, e, 0)
    e = np.clip(e, -127, 127)
    scale = np.ldexp(1.0, e)[:, :, None]
    q = blk / scale
    code = e2m1_encode(np.abs(q)) | np.where(q < 0, 8, 0).astype(np.uint8)
    code = code.reshape(rows, K)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    scales = (e + 127).astype(np.uint8)
    return packed, scales


def _ksteps(dtype, K):
    return -(-K // 128) if dtype == MXFP4 else K // 32


def _matrix_bytes(dtype, rows, K):
    if dtype == F32:
        return 4 * rows * K
    if dtype == BF16:
        return 2 * rows * K
    return rows // 16 * _ksteps(dtype, K) * 1024


def _scale_blocks(K):
    """16-step blocks of MXFP4 scales per row tile."""
    return -(-_ksteps(MXFP4, K) // 16)


def _scale_bytes(rows, K):
    return rows // 16 * _scale_blocks(K) * 1024


def slot_offsets(dtype: int, H: int, I: int) -> dict:
    """Byte offsets of the parts of one expert slot (w13, w2, s13, s2, total)."""
    o = {"w13": 0, "w2": _matrix_bytes(dtype, 2 * I, H)}
    end = o["w2"] + _matrix_bytes(dtype, H, I)
    if dtype == MXFP4:
        o["s13"] = end
        o["s2"] = end + _scale_bytes(2 * I, H)
        end = o["s2"] + _scale_bytes(H, I)
    o["total"] = end
    return o


def expert_bytes(dtype: int, H: int, I: int) -> int:
    """Bytes of one expert's slot in the documented layout."""
    if dtype == MXFP4:
        assert H % 32 == 0 and I % 32 == 0
    return slot_offsets(dtype, H, I)["total"]


def _tile_bf16(m):
    R, K = m.shape
    b = bf16_bits(np.asarray(m, np.float32))
    return b.reshape(R // 16, 16, K // 32, 4, 8).transpose(0, 2, 3, 1, 4).ravel().view(np.uint8)


def _tile_mx(m):
    R, K = m.shape
    codes, scales = mx_quantize(m)
    nk = _ksteps(MXFP4, K)
    blocks = codes.reshape(R, K // 32, 16)
    pad_c = np.zeros((R, nk * 4, 16), np.uint8)
    pad_c[:, : K // 32] = blocks
    pad_s = np.zeros((R, nk * 4), np.uint8)
    pad_s[:, : K // 32] = scales
    tc = pad_c.reshape(R // 16, 16, nk, 4, 16).transpose(0, 2, 3, 1, 4).ravel()
    # scales: per row tile, blocks of 16 column steps; inside a block fragment
    # f = 16*group + row%16 owns 16 bytes, byte i = its scale at step 16*block + i
    nb = _scale_blocks(K)
    pad_s2 = np.zeros((R, nb * 16 * 4), np.uint8)
    pad_s2[:, : nk * 4] = pad_s
    ts = pad_s2.reshape(R // 16, 16, nb, 16, 4).transpose(0, 2, 4, 1, 3).ravel()
    return tc, ts


def _interleave_w13(w_gate, w_up):
    I, H = w_gate.shape
    assert I % 8 == 0
    w = np.empty((2 * I, H), dtype=np.float64)
    v = w.reshape(I // 8, 16, H)
    v[:, :8] = np.asarray(w_gate, np.float64).reshape(I // 8, 8, H)
    v[:, 8:] = np.asarray(w_up, np.float64).reshape(I // 8, 8, H)
    return w


def pack_expert(dtype: int, w_gate, w_up, w_down) -> np.ndarray:
    """Encode float matrices Wg [I][H], Wu [I][H], Wd [H][I] into one slot (uint8)."""
    w_gate, w_up, w_down = (np.asarray(a) for a in (w_gate, w_up, w_down))
    I, H = w_gate.shape
    if dtype == F32:
        w13 = np.concatenate([w_gate, w_up], axis=0)
        parts = [w13.astype(np.float32).ravel().view(np.uint8), w_down.astype(np.float32).ravel().view(np.uint8)]
    elif dtype == BF16:
        w13 = _interleave_w13(w_gate, w_up).astype(np.float32)
        parts = [_tile_bf16(w13), _tile_bf16(w_down.astype(np.float32))]
    elif dtype == MXFP4:
        c13, s13 = _tile_mx(_interleave_w13(w_gate, w_up))
        c2, s2 = _tile_mx(np.asarray(w_down, np.float64))
        parts = [c13, c2, s13, s2]
    else:
        raise ValueError(dtype)
    out = np.concatenate(parts).astype(np.uint8)
    assert out.size == expert_bytes(dtype, H, I)
    return out


def random_expert(dtype: int, H: int, I: int, g: np.random.Generator, std: float = 0.02) -> np.ndarray:
    """One expert with N(0, std) weights, encoded into its slot bytes."""
    wg = (g.standard_normal((I, H)) * std).astype(np.float32)
    wu = (g.standard_normal((I, H)) * std).astype(np.float32)
    wd = (g.standard_normal((H, I)) * std).astype(np.float32)
    return pack_expert(dtype, wg, wu, wd)


def encode_activations(dtype: int, x_f32) -> np.ndarray:
    """Token activations in the layer's activation format: f32 for f32 weights,
    bf16 bits otherwise (MXFP4 layers take bf16 activations)."""
    x_f32 = np.ascontiguousarray(x_f32, dtype=np.float32)
    if dtype == F32:
        return x_f32
    return bf16_bits(x_f32)


# ----------------------------------------------------------------------------
# Bulk generation on the GPU with torch (large pools).  Same encodings as above.
# ----------------------------------------------------------------------------

def torch_bf16_expert_pool(n_experts: int, H: int, I: int, seed: int, device, std: float = 0.02, chunk: int = 16):
    """uint8 tensor [n_experts][expert_bytes] of bf16 experts with N(0, std) weights.

    Every element is an independent draw, so the flat order of the draws does not
    matter for the layout; torch's float32 -> bfloat16 conversion rounds to
    nearest even.  Experts are drawn `chunk` at a time.
    """
    import torch
    nb = expert_bytes(BF16, H, I)
    out = torch.empty((n_experts, nb), dtype=torch.uint8, device=device)
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    for e0 in range(0, n_experts, chunk):
        e1 = min(n_experts, e0 + chunk)
        w = torch.randn((e1 - e0, 3 * H * I), generator=g, device=device, dtype=torch.float32) * std
        out[e0:e1].copy_(w.to(torch.bfloat16).view(torch.uint8))
    return out


def torch_mx_quantize_flat(w):
    """torch float32 vector (len % 32 == 0) -> (codes uint8 [len/2], scales uint8 [len/32]).

    Same rule as mx_quantize, applied to consecutive 32-element blocks.
    """
    import torch
    blk = w.double().reshape(-1, 32)
    amax = blk.abs().amax(dim=1)
    safe = torch.where(amax > 0, amax, torch.ones_like(amax))
    e = torch.floor(torch.log2(safe)).to(torch.int64) - 2
    e = torch.where(amax > 0, e, torch.zeros_like(e)).clamp(-127, 127)
    q = blk / torch.ldexp(torch.ones_like(amax), e)[:, None]
    m = q.abs()
    code = torch.zeros(m.shape, dtype=torch.uint8, device=w.device)
    for i, b in enumerate(_E2M1_MID.tolist()):
        code += (m > b).to(torch.uint8)
        if i % 2 == 1:
            code += (m == b).to(torch.uint8)
    code |= torch.where(q < 0, 8, 0).to(torch.uint8)
    code = code.reshape(-1)
    packed = code[0::2] | (code[1::2] << 4)
    return packed, (e + 127).to(torch.uint8)


def torch_mxfp4_expert_pool(n_experts: int, H: int, I: int, seed: int, device, std: float = 0.02, chunk: int = 4):
    """uint8 tensor [n_experts][expert_bytes] of MXFP4 experts with N(0, std) weights.

    Every element is an independent draw, so consecutive 32-element blocks of the
    flat draw vector can be placed at consecutive fragments of the tiled layout
    (fragment order: matrix, row tile, column step, fragment); each scale is then
    moved from that order to its place in the blocked scale layout.  Experts are
    drawn `chunk` at a time.
    """
    import torch
    assert H % 2048 == 0 and I % 2048 == 0, "bulk MXFP4 pools need 16-step multiples of K (no padding)"
    nb = expert_bytes(MXFP4, H, I)
    n = 3 * H * I
    mats = [(2 * I, H), (H, I)]  # W13, W2: (rows, K)
    out = torch.empty((n_experts, nb), dtype=torch.uint8, device=device)
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    for e0 in range(0, n_experts, chunk):
        e1 = min(n_experts, e0 + chunk)
        ne = e1 - e0
        w = torch.randn(ne * n, generator=g, device=device, dtype=torch.float32) * std
        c, s = torch_mx_quantize_flat(w)
        out[e0:e1, : n // 2].copy_(c.view(ne, n // 2))
        s = s.view(ne, n // 32)
        pos, off = n // 2, 0
        for rows, K in mats:
            rt, nk = rows // 16, K // 128
            cnt = rt * nk * 64
            blk = s[:, off:off + cnt].reshape(ne, rt, nk // 16, 16, 64).transpose(3, 4)
            out[e0:e1, pos:pos + cnt].copy_(blk.reshape(ne, cnt))
            pos += cnt
            off += cnt
    return out
