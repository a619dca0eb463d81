"""Storage formats used on the hot path, decoded and encoded in float64.

Test infrastructure (see the package docstring).  The pages fix only the formats'
names: "DeepSeek-V4 深度分析报告" section 2.1 / "其他注意力技术细节" (RoPE dims kept in
BF16, the other dims in FP8, the Lightning Indexer computing in FP4), its section 3.4
(MXFP4 on the CSA QK path) and the stuffyNLP review's paragraph on MXFP4 and the FP8
1x128 / 128x128 scheme kept from DeepSeek-V3.  The bit layouts are the public OCP
definitions:

* bf16: 1 sign, 8 exponent (bias 127), 7 mantissa bits; round-to-nearest-even.
* fp8 e4m3fn (OCP 8-bit floating point v1.0): bias 7, no infinities, S.1111.111 = NaN,
  max normal 448, min normal 2^-6, min subnormal 2^-9.
* e2m1 (OCP Microscaling v1.0 FP4 element): bias 1, values 0, 0.5, 1, 1.5, 2, 3, 4, 6.
* e8m0 (OCP MX shared scale): 2^(code-127), code 0xFF = NaN.

Readings (the pages are silent on the recipe):
* FP8 1x128 (KV rows): the first d_n = D - 64 dims are cut into 128-wide blocks
  (448 = 128+128+128+64); scale_b = fp32(amax_b / 448); code = RNE_e4m3(x / scale_b),
  saturating at +-448; an all-zero block gets scale 0 and zero codes.  The trailing
  64 RoPE dims are stored as bf16.  The same recipe over all D dims (no bf16 tail) is
  the fp8 alternative for indexer queries and keys.
* MXFP4: 32-element blocks; shared exponent E = floor(log2(amax)) - 2 (2 = emax of e2m1),
  clamped to [-127, 127]; element = RNE_e2m1(x / 2^E) saturating at +-6; amax == 0
  gives E = -127 and zero codes.  Packing: element 2i in the low nibble of byte i.
"""

import numpy as np

# ----------------------------------------------------------------------------- rounding


def round_rne(x, mant_bits, emin, maxval=None, saturate=False):
    """Round float64 values to a binary format with `mant_bits` stored mantissa bits
    and minimum normal exponent `emin`, ties to even.  Exact: x / ulp is a power-of-two
    scaling and np.rint rounds half to even.  Out-of-range results saturate to
    +-maxval or become +-inf."""
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    _, E = np.frexp(np.where(ax > 0, ax, 1.0))  # ax = f * 2^E, f in [0.5, 1)
    e = np.maximum(E - 1, emin)
    ulp = np.ldexp(1.0, e - mant_bits)
    r = np.rint(x / ulp) * ulp
    r = np.where(ax > 0, r, x)  # keeps +-0
    if maxval is not None:
        over = np.abs(r) > maxval
        if saturate:
            r = np.where(over, np.copysign(maxval, x), r)
        else:
            r = np.where(over, np.copysign(np.inf, x), r)
    return r


# ----------------------------------------------------------------------------- bf16

BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def bf16_round(x):
    return round_rne(x, 7, -126, BF16_MAX, saturate=False)


def encode_bf16(x):
    """float64 -> bf16 bit patterns (uint16), RNE.  The rounded value is exactly
    representable in float32, so its top 16 bits are the bf16 pattern."""
    r = bf16_round(x).astype(np.float32)
    return (r.view(np.uint32) >> 16).astype(np.uint16)


def decode_bf16(bits):
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------- fp8 e4m3fn

E4M3_MAX = 448.0


def _e4m3fn_value(code):
    s = (code >> 7) & 1
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return np.nan
    if e == 0:
        v = (m / 8.0) * 2.0 ** -6
    else:
        v = (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -v if s else v


E4M3FN_TABLE = np.array([_e4m3fn_value(c) for c in range(256)], dtype=np.float64)
_E4M3_POS = E4M3FN_TABLE[:127]  # codes 0..126: 0 .. 448, strictly increasing


def decode_e4m3fn(codes):
    return E4M3FN_TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3fn_round(x):
    return round_rne(x, 3, -6, E4M3_MAX, saturate=True)


def encode_e4m3fn(x):
    """float64 -> e4m3fn codes (uint8), RNE with saturation at +-448.  NaN inputs are
    not expected (they would map to 0x7F)."""
    x = np.asarray(x, dtype=np.float64)
    r = e4m3fn_round(x)
    mag = np.abs(r)
    idx = np.searchsorted(_E4M3_POS, mag)
    idx = np.minimum(idx, 126)
    assert np.all(_E4M3_POS[idx] == mag), "rounded value not on the e4m3fn grid"
    code = idx.astype(np.uint8)
    code = np.where(np.signbit(r), code | 0x80, code).astype(np.uint8)
    return code


# ----------------------------------------------------------------------------- fp4 e2m1 / e8m0

E2M1_MAX = 6.0


def _e2m1_value(code):
    s = (code >> 3) & 1
    e = (code >> 1) & 0x3
    m = code & 0x1
    if e == 0:
        v = m * 0.5
    else:
        v = (1.0 + m / 2.0) * 2.0 ** (e - 1)
    return -v if s else v


E2M1_TABLE = np.array([_e2m1_value(c) for c in range(16)], dtype=np.float64)
_E2M1_POS = E2M1_TABLE[:8]


def decode_e2m1(codes):
    return E2M1_TABLE[np.asarray(codes, dtype=np.uint8) & 0xF]


def e2m1_round(x):
    return round_rne(x, 1, 0, E2M1_MAX, saturate=True)


def encode_e2m1(x):
    r = e2m1_round(np.asarray(x, dtype=np.float64))
    mag = np.abs(r)
    idx = np.searchsorted(_E2M1_POS, mag)
    idx = np.minimum(idx, 7)
    assert np.all(_E2M1_POS[idx] == mag), "rounded value not on the e2m1 grid"
    return np.where(np.signbit(r), idx | 0x8, idx).astype(np.uint8)


def decode_e8m0(codes):
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    v = np.ldexp(1.0, c - 127)
    return np.where(c == 255, np.nan, v)


# ----------------------------------------------------------------------------- block formats

KV_BLOCK = 128
MX_BLOCK = 32


def kv_split_blocks(d_n):
    """Column ranges of the 1x128 scale blocks over the first d_n dims."""
    return [(s, min(s + KV_BLOCK, d_n)) for s in range(0, d_n, KV_BLOCK)]


def quant_kv_split(x, rope_dims=64):
    """Rows [..., D] float64 -> (codes uint8 [..., D-r], scales float32 [..., nblk],
    rope bf16 bits uint16 [..., r])."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    d_n = D - rope_dims
    blocks = kv_split_blocks(d_n)
    codes = np.zeros(x.shape[:-1] + (d_n,), dtype=np.uint8)
    scales = np.zeros(x.shape[:-1] + (len(blocks),), dtype=np.float32)
    for b, (lo, hi) in enumerate(blocks):
        blk = x[..., lo:hi]
        amax = np.max(np.abs(blk), axis=-1)
        sc = (amax / E4M3_MAX).astype(np.float32)
        scales[..., b] = sc
        sc64 = sc.astype(np.float64)[..., None]
        safe = np.where(sc64 > 0, sc64, 1.0)
        q = np.where(sc64 > 0, blk / safe, 0.0)
        codes[..., lo:hi] = encode_e4m3fn(q)
    rope = encode_bf16(x[..., d_n:])
    return codes, scales, rope


def dequant_kv_split(codes, scales, rope_bits):
    codes = np.asarray(codes, dtype=np.uint8)
    d_n = codes.shape[-1]
    out = np.empty(codes.shape[:-1] + (d_n + np.asarray(rope_bits).shape[-1],), dtype=np.float64)
    for b, (lo, hi) in enumerate(kv_split_blocks(d_n)):
        out[..., lo:hi] = decode_e4m3fn(codes[..., lo:hi]) * np.asarray(scales, dtype=np.float64)[..., b:b + 1]
    out[..., d_n:] = decode_bf16(rope_bits)
    return out


def quant_fp8_b128(x):
    """Rows [..., D] float64 -> (codes uint8 [..., D], scales float32 [..., ceil(D/128)]):
    the FP8 1x128 recipe of the KV rows applied to every dim (no bf16 tail)."""
    codes, scales, _ = quant_kv_split(x, 0)
    return codes, scales


def dequant_fp8_b128(codes, scales):
    codes = np.asarray(codes, dtype=np.uint8)
    return dequant_kv_split(codes, scales, np.zeros(codes.shape[:-1] + (0,), dtype=np.uint16))


def quant_mxfp4(x):
    """Rows [..., D] float64 (D % 32 == 0) -> (packed uint8 [..., D/2], e8m0 uint8 [..., D/32])."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    assert D % MX_BLOCK == 0
    blk = x.reshape(x.shape[:-1] + (D // MX_BLOCK, MX_BLOCK))
    amax = np.max(np.abs(blk), axis=-1)
    _, E = np.frexp(np.where(amax > 0, amax, 1.0))
    shared = np.where(amax > 0, (E - 1) - 2, -127)
    shared = np.clip(shared, -127, 127)
    scaled = blk / np.ldexp(1.0, shared)[..., None]
    codes = encode_e2m1(scaled).reshape(x.shape)
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    return packed, (shared + 127).astype(np.uint8)


def unpack_e2m1(packed):
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed & 0xF
    out[..., 1::2] = packed >> 4
    return out


def dequant_mxfp4(packed, scales):
    codes = unpack_e2m1(packed)
    vals = decode_e2m1(codes)
    D = vals.shape[-1]
    s = decode_e8m0(scales)
    return (vals.reshape(vals.shape[:-1] + (D // MX_BLOCK, MX_BLOCK)) * s[..., None]).reshape(vals.shape)
