"""Plain CPU oracle for the W4A16 weight-only linear layer.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module. The product
path (the HIP library and its Python binding) never touches it, and it shares
no code with that path: its own converters, its own quantiser, its own
implementation of the packed device layout.

What it computes, and where the method is stated:

* The format. Weights are kept as small integers with a scale, and usually a
  zero-point, per group; the kernel unpacks them and rebuilds approximate
  FP16/BF16 values just before the multiply, while activations stay 16-bit and
  accumulation stays in higher precision ("Weight-Only Quantisation", klaylearn
  glossary: the definition paragraphs and the first FAQ answer; "Weight-Only
  Quantization Explained", multigrid.ai: "What W4A16 actually names").
* The quantiser. Round-to-nearest of w/scale ("Quantization Is Not a Zip File",
  zhuai.tech, section 3 "The core idea: local structure, not global rounding"),
  applied per group of 32/64/128 consecutive weights ("Block locality" in that
  same section; 256 as well, the super-block size the K-quant row of the table
  in that page's "How to read common GGUF quantization names" gives), with an asymmetric zero-point and the reconstruction
  (q - zero) * scale ("Comparison of Quantization Methods: INT8 vs GPTQ vs AWQ
  vs GGUF", instagit, "Practical Code Examples", the zero-point example).
* The metadata width. 4 + 20/group bits per weight: a 16-bit scale and a 4-bit
  zero per group, which gives the 4.156 bits/weight printed for group 128
  ("Weight-Only Quantization Explained", "The memory arithmetic").

* The symmetric variants. No zero-point: q = round(w / s) clamped to the signed
  range [-2**(b-1), 2**(b-1) - 1] and w_hat = q * s, with s = max|w| / (2**(b-1) - 1)
  (the symmetric INT8 scheme of the instagit comparison page, "INT8: Symmetric
  Integer Quantization" and "Practical Code Examples", applied per group as the
  "Classic blocks" row of the zhuai.tech table in "How to read common GGUF
  quantization names" does: integer codes plus one scale per block; INT8 or
  INT4 weights with FP16/BF16 activations are both weight-only schemes:
  "Weight-Only Quantisation", definition). 4-bit (sym4) and 8-bit (sym8, W8A16)
  codes are stored offset by 2**(b-1), so the shared reconstruction
  s * (code - zero) holds with a fixed zero of 8 or 128 that is never stored.

* The quality report (MSE, SNR, cosine, max error) of the error-analysis
  routine the instagit page lists, and AWQ's run-time half (activations
  multiplied by the reciprocal of the factors the weights were scaled up by),
  both at the end of this module.

Readings where the pages are silent (each also listed in the design notes):
  * range includes zero: lo = min(0, min w), hi = max(0, max w);
  * scale s = fp16_rne((hi - lo) / 15) computed in fp32; a zero scale becomes
    the smallest positive fp16 (2**-24);
  * zero z = clamp(rint(-lo / s), 0, 15); code q = clamp(rint(w / s) + z, 0, 15);
    rint rounds half to even; every quantiser operation is IEEE fp32 (the
    precision the kernel takes the same integer decision in);
  * symmetric: s = fp16_rne(max|w| / qmax) in fp32 (qmax = 7 or 127, zero
    scale -> 2**-24), code = clamp(rint(w / s), -qmax-1, qmax) + qmax + 1;
  * groups of 32, 64, 128 or 256 consecutive weights along K;
  * dequantised weight w_hat = s * (q - z) is exact in fp64 here;
  * y = x @ w_hat^T accumulated in fp64.

Weights must be finite with |w| < 2**18 so that the fp16 scale is finite.
"""
from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# 16-bit float conversions, bit level (round to nearest, ties to even).
# The pages name fp16/bf16 as the activation and reconstruction types
# ("Weight-Only Quantisation", definition); the instagit page's
# "Implementation Architecture" lists bit-level float converters as the first
# building block. Written out here from the IEEE 754 binary16 / bfloat16
# definitions, not taken from any library.
# ---------------------------------------------------------------------------


def _rne_shift_right(v: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Round the non-negative integers v / 2**s to nearest, ties to even (s >= 1)."""
    v = v.astype(np.uint64)
    s = s.astype(np.uint64)
    q = v >> s
    rem = v - (q << s)
    half = np.left_shift(np.uint64(1), s - np.uint64(1))
    up = (rem > half) | ((rem == half) & ((q & np.uint64(1)) == 1))
    return q + up.astype(np.uint64)


def f32_to_f16_bits(a) -> np.ndarray:
    """IEEE binary32 -> binary16 bits, RNE, subnormals kept, overflow -> inf."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    sign = (u >> np.uint64(31)) << np.uint64(15)
    exp = ((u >> np.uint64(23)) & np.uint64(0xFF)).astype(np.int64)
    man = u & np.uint64(0x7FFFFF)
    out = np.zeros(a.shape, dtype=np.uint64)

    is_nan = (exp == 255) & (man != 0)
    is_inf = (exp == 255) & (man == 0)
    finite = exp < 255
    e = exp - 127                      # unbiased exponent of a normal fp32 value
    sig = man | np.uint64(1 << 23)     # 24-bit significand, value = sig * 2**(e-23)

    # Result is a normal fp16 (or rounds up to inf): exponent field e + 15 in [1, 30].
    normal = finite & (exp > 0) & (e >= -14)
    # value in units of 2**(e-10): keep 11 significant bits
    r = _rne_shift_right(sig, np.full(sig.shape, 13))          # 11 or 12 bits after rounding
    carry = r >> np.uint64(11)                                  # 1 if rounding overflowed to 2**11
    r_n = np.where(carry == 1, r >> np.uint64(1), r)
    e_n = e + carry.astype(np.int64)
    h_norm = (((e_n + 15).astype(np.uint64)) << np.uint64(10)) | (r_n & np.uint64(0x3FF))
    h_norm = np.where(e_n > 15, np.uint64(0x7C00), h_norm)     # overflow -> inf

    # Result is subnormal (or zero): value in units of 2**-24 is sig * 2**(e-23+24).
    sub = finite & (exp > 0) & (e < -14)
    shift = np.clip(-(e + 1), 1, 40)                            # e+1 <= -14  ->  shift >= 14
    h_sub = np.where(shift >= 26, np.uint64(0), _rne_shift_right(sig, shift))
    # (a result of 1024 units is the smallest normal, 0x0400, which is the same bits)

    out = np.where(normal, h_norm, out)
    out = np.where(sub, h_sub, out)
    # fp32 zeros and fp32 subnormals (exp == 0) are below 2**-126: they round to zero.
    out = np.where(is_inf, np.uint64(0x7C00), out)
    out = np.where(is_nan, np.uint64(0x7E00), out)
    return (out | sign).astype(np.uint16)


def f16_bits_to_f64(h) -> np.ndarray:
    """binary16 bits -> exact float64 value."""
    h = np.asarray(h, dtype=np.uint16).astype(np.int64)
    sign = np.where((h >> 15) & 1, -1.0, 1.0)
    exp = (h >> 10) & 0x1F
    man = h & 0x3FF
    mag = np.where(exp == 0, np.ldexp(man.astype(np.float64), -24),
                   np.ldexp((man + 1024).astype(np.float64), (exp - 25).astype(np.int64)))
    mag = np.where(exp == 31, np.where(man == 0, np.inf, np.nan), mag)
    return sign * mag


def f16_bits_to_f32(h) -> np.ndarray:
    """binary16 bits -> float32 (exact: every binary16 value is a binary32 value)."""
    return f16_bits_to_f64(h).astype(np.float32)


def f32_to_bf16_bits(a) -> np.ndarray:
    """IEEE binary32 -> bfloat16 bits, RNE (the upper 16 bits, rounded)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    is_nan = ((u >> np.uint64(23)) & np.uint64(0xFF) == 0xFF) & ((u & np.uint64(0x7FFFFF)) != 0)
    upper = u >> np.uint64(16)
    rem = u & np.uint64(0xFFFF)
    up = (rem > 0x8000) | ((rem == 0x8000) & ((upper & np.uint64(1)) == 1))
    r = upper + up.astype(np.uint64)          # carries into the exponent, max finite -> inf
    r = np.where(is_nan, upper | np.uint64(0x40), r)
    return r.astype(np.uint16)


def bf16_bits_to_f64(b) -> np.ndarray:
    """bfloat16 bits -> exact float64 value (bf16 is the top half of a binary32)."""
    b = np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def act_bits_to_f64(bits, dtype: str) -> np.ndarray:
    if dtype == "f16":
        return f16_bits_to_f64(bits)
    if dtype == "bf16":
        return bf16_bits_to_f64(bits)
    raise ValueError(dtype)


def out_round_bits(y64, dtype: str) -> np.ndarray:
    """Round fp64 results to the output type as the kernel does: to fp32 first, then RNE."""
    y32 = np.asarray(y64, dtype=np.float64).astype(np.float32)
    return f32_to_f16_bits(y32) if dtype == "f16" else f32_to_bf16_bits(y32)


# ---------------------------------------------------------------------------
# Byte accounting ("Weight-Only Quantization Explained", "The memory
# arithmetic": 4.156 bits per weight at group 128, 26.0 GB vs 6.75 GB for 13e9
# weights; "Quantization Is Not a Zip File", section 2: 2N / 1N / 0.5N bytes).
# ---------------------------------------------------------------------------


def bits_per_weight(group: int, scale_bits: int = 16, zero_bits: int = 4, code_bits: int = 4) -> float:
    """Storage per weight: the code plus the group's scale and zero spread over the group."""
    return code_bits + (scale_bits + zero_bits) / group


FORMATS = ("asym4", "sym4", "sym8", "kq4")


def code_bits(fmt: str) -> int:
    if fmt not in FORMATS:
        raise ValueError(fmt)
    return 8 if fmt == "sym8" else 4


def format_bits_per_weight(group: int, fmt: str = "asym4") -> float:
    """Storage per weight of a format: the code, the fp16 scale, and the 4-bit
    zero-point only where the format stores one. kq4: 4-bit codes plus a 16-byte
    record per 256 weights (4.5 bits)."""
    if fmt == "kq4":
        return 4 + 8 * KQ_RECORD_BYTES / KQ_SUPER
    return bits_per_weight(group, code_bits=code_bits(fmt), zero_bits=4 if fmt == "asym4" else 0)


def packed_bytes(N: int, K: int, group: int, fmt: str = "asym4"):
    """(qweight, scales, zeros) algorithmic byte counts: one code per weight, one fp16
    scale per (group, output column), and for asym4 one 4-bit zero per (group, column).
    kq4 (group 256): one 16-byte record per (super-block, column), no zeros."""
    G = K // group
    if fmt == "kq4":
        return N * K // 2, KQ_RECORD_BYTES * G * N, 0
    return (N * K * code_bits(fmt)) // 8, 2 * G * N, (G * N) // 2 if fmt == "asym4" else 0


def model_bytes(n_weights: float, bits: float) -> float:
    return n_weights * bits / 8


# ---------------------------------------------------------------------------
# Groupwise asymmetric round-to-nearest quantiser.
# Rounding step: "Quantization Is Not a Zip File", section 3 (q = round(w/scale),
# w_hat = scale * q). Groups of 32/64/128 along K with their own scale: same
# section, "Block locality". Zero-point and (q - zero) * scale reconstruction:
# instagit comparison page, "Practical Code Examples" (asymmetric example).
# ---------------------------------------------------------------------------

F16_MIN_SUBNORMAL_BITS = np.uint16(0x0001)   # 2**-24


GROUPS = (32, 64, 128, 256)


def quantize_groupwise(w, group: int, fmt: str = "asym4"):
    """Quantise fp32 weights w [N][K] in groups of `group` consecutive k.

    Returns (codes u8 [N][K], scale_bits u16 [G][N], zeros u8 [G][N]); for the
    symmetric formats the zeros are the fixed offset (8 or 128), not stored on
    the device. Every step is an IEEE binary32 operation (division, never a
    reciprocal).
    """
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    if group not in GROUPS or K % group != 0:
        raise ValueError("group must be 32/64/128/256 and divide K")
    if fmt not in FORMATS or fmt == "kq4":
        raise ValueError(f"unknown format {fmt} (kq4: quantize_kquant)")
    if not np.all(np.isfinite(w)) or np.max(np.abs(w), initial=0.0) >= 2.0 ** 18:
        raise ValueError("weights must be finite with |w| < 2**18")
    G = K // group
    wg = w.reshape(N, G, group)
    if fmt != "asym4":
        return _quantize_symmetric(wg, code_bits(fmt))
    zero = np.float32(0.0)
    # 1. range of the group, widened to include zero
    lo = np.minimum(wg.min(axis=2), zero)                       # [N][G] fp32
    hi = np.maximum(wg.max(axis=2), zero)
    # 2. scale: fp32 (hi - lo) / 15, rounded once to fp16; zero -> smallest subnormal
    s32 = (hi - lo) / np.float32(15.0)
    s_bits = f32_to_f16_bits(s32)
    s_bits = np.where(s_bits == 0, F16_MIN_SUBNORMAL_BITS, s_bits).astype(np.uint16)
    s = f16_bits_to_f32(s_bits)                                  # exact widening
    # 3. zero-point: the code that reconstructs to (about) lo
    z = np.clip(np.rint(-lo / s), 0, 15).astype(np.int32)
    # 4. codes: round(w / s) + z, clamped to the 4-bit range
    r = np.rint(wg / s[:, :, None]).astype(np.int32)
    q = np.clip(r + z[:, :, None], 0, 15).astype(np.uint8)
    return (q.reshape(N, K), np.ascontiguousarray(s_bits.T), np.ascontiguousarray(z.T.astype(np.uint8)))


def _quantize_symmetric(wg, bits: int):
    """Symmetric groupwise round-to-nearest of wg [N][G][group] with b-bit codes:
    s = max|w| / (2**(b-1) - 1), q = clamp(rint(w / s), -2**(b-1), 2**(b-1) - 1),
    stored as q + 2**(b-1)."""
    N, G, group = wg.shape
    qmax = (1 << (bits - 1)) - 1
    off = qmax + 1
    # 1. the group's largest magnitude (exact in fp32)
    amax = np.abs(wg).max(axis=2)
    # 2. scale: fp32 amax / qmax rounded once to fp16; zero -> smallest subnormal
    s_bits = f32_to_f16_bits(amax / np.float32(qmax))
    s_bits = np.where(s_bits == 0, F16_MIN_SUBNORMAL_BITS, s_bits).astype(np.uint16)
    s = f16_bits_to_f32(s_bits)
    # 3. codes: round(w / s) in the signed range, offset to unsigned
    q = np.clip(np.rint(wg / s[:, :, None]).astype(np.int32), -off, qmax) + off
    zeros = np.full((G, N), off, dtype=np.uint8)
    return (q.astype(np.uint8).reshape(N, G * group), np.ascontiguousarray(s_bits.T), zeros)


def dequantize(codes, scale_bits, zeros, group: int) -> np.ndarray:
    """w_hat [N][K] = s * (q - z), exact in fp64."""
    codes = np.asarray(codes, dtype=np.uint8)
    N, K = codes.shape
    G = K // group
    s = f16_bits_to_f64(scale_bits).T                           # [N][G]
    z = np.asarray(zeros, dtype=np.int64).T                     # [N][G]
    d = codes.reshape(N, G, group).astype(np.int64) - z[:, :, None]
    return (d.astype(np.float64) * s[:, :, None]).reshape(N, K)


# ---------------------------------------------------------------------------
# Packing. The pages require the data to stay packed until the kernel
# ("Quantization Is Not a Zip File", section 8) and say the packing layout is
# one of the things that decides speed ("Weight-Only Quantisation",
# definition). The layouts themselves are this library's own; the device
# layout is written out here independently from its specification:
#
#   qweight: rows in blocks of 16 (the last block may hold fewer rows,
#   rows_b = min(16, N - 16 b)); K in chunks of 32 weights (C = K/32 chunks)
#   and columns of 4 chunks (the last column may hold fewer, nc = min(4,
#   C - 4t)). A chunk of one row is 4 dwords; dword d = (k % 32) // 8 holds
#   k = 32c + 8d + i, i = 0..7, in nibble p = i // 2 + 4 * (i % 2) (even k in
#   the low half-word, odd k in the high half-word). Byte offset of dword d of
#   chunk c = 4t + j of row n = 16b + r:
#       16*b*(K/2) + t*rows_b*64 + d*(rows_b*nc*4) + r*(nc*4) + j*4.
#   So for a full column the 16 rows x 4 dword positions form one contiguous
#   KiB in which the 16 bytes at d*256 + r*16 are dword d of the column's four
#   chunks of row r. Dwords are little-endian.
#   Metadata (layout 3), one row after another so that a row's metadata for a
#   run of K is contiguous: G = K/group groups per row, padded to G8 (the next
#   multiple of 8; padded slots hold 0).
#   scales: fp16 bits [N][G8] (group g of row n is element n*G8 + g).
#   zeros: u32 words [N][G8/8]; group g of row n is nibble g % 8 of word
#   n*(G8/8) + g // 8 (little-endian words, nibble i at bits 4i..4i+3).
#   K-quant super-block records: [N][K/256] of 16 bytes.
#   8-bit codes (sym8) are two 4-bit planes, each in the qweight layout above:
#   the low nibbles of every code first (N*K/2 bytes), then the high nibbles.
#   The symmetric formats store no zero words.
# ---------------------------------------------------------------------------


def _device_nibble_index(N: int, K: int) -> np.ndarray:
    """Nibble position in the packed qweight stream of every (n, k), shape [N][K]."""
    n = np.arange(N, dtype=np.int64)[:, None]
    k = np.arange(K, dtype=np.int64)[None, :]
    C = K // 32
    b = n // 16
    r = n % 16
    rows_b = np.minimum(16, N - 16 * b)
    c = k // 32
    t = c // 4
    j = c % 4
    nc = np.minimum(4, C - 4 * t)
    d = (k % 32) // 8
    i = k % 8
    p = i // 2 + 4 * (i % 2)
    byte_off = 16 * b * (K // 2) + t * rows_b * 64 + d * (rows_b * nc * 4) + r * (nc * 4) + j * 4
    dword = byte_off // 4
    return dword * 8 + p


def pack_device(codes, fmt: str = "asym4") -> np.ndarray:
    """codes u8 [N][K] -> packed qweight bytes (uint8, N*K/2 or N*K for sym8) in the
    device layout."""
    codes = np.asarray(codes, dtype=np.uint8)
    if code_bits(fmt) == 8:
        return np.concatenate([pack_device(codes & np.uint8(0xF)), pack_device(codes >> np.uint8(4))])
    N, K = codes.shape
    if N % 8 or K % 32:
        raise ValueError("N % 8 == 0 and K % 32 == 0 required")
    nib = np.empty(N * K, dtype=np.uint8)
    nib[_device_nibble_index(N, K).ravel()] = codes.ravel()
    # nibble t sits in byte t // 2, low nibble when t is even (little-endian dwords)
    return (nib[0::2] | (nib[1::2] << 4)).astype(np.uint8)


def unpack_device(qweight, N: int, K: int, fmt: str = "asym4") -> np.ndarray:
    """Inverse of pack_device: packed bytes -> codes u8 [N][K]."""
    qb = np.asarray(qweight, dtype=np.uint8).ravel()
    if code_bits(fmt) == 8:
        half = N * K // 2
        return unpack_device(qb[:half], N, K) | (unpack_device(qb[half:], N, K) << np.uint8(4))
    nib = np.empty(2 * qb.size, dtype=np.uint8)
    nib[0::2] = qb & 0xF
    nib[1::2] = qb >> 4
    return nib[_device_nibble_index(N, K)]


def pack_zeros(zeros) -> np.ndarray:
    """zeros u8 [G][N] -> u32 [G][N/8], nibble n % 8 of word n // 8 (canonical form)."""
    z = np.asarray(zeros, dtype=np.uint32)
    G, N = z.shape
    zz = z.reshape(G, N // 8, 8)
    word = np.zeros((G, N // 8), dtype=np.uint32)
    for t in range(8):
        word |= zz[:, :, t] << np.uint32(4 * t)
    return word


def unpack_zeros(words, G: int, N: int) -> np.ndarray:
    w = np.asarray(words, dtype=np.uint32).reshape(G, N // 8)
    out = np.empty((G, N // 8, 8), dtype=np.uint8)
    for t in range(8):
        out[:, :, t] = (w >> np.uint32(4 * t)) & np.uint32(0xF)
    return out.reshape(G, N)


def padded_groups(G: int) -> int:
    """G8: metadata slots per row, the group count rounded up to a multiple of 8."""
    return -(-G // 8) * 8


def pack_scales_device(scale_bits, group: int) -> np.ndarray:
    """scale bits [G][N] -> device order [N][G8] (uint16), padded slots 0."""
    s = np.asarray(scale_bits, dtype=np.uint16)
    G, N = s.shape
    out = np.zeros((N, padded_groups(G)), dtype=np.uint16)
    out[:, :G] = s.T
    return out


def pack_zeros_device(zeros, group: int) -> np.ndarray:
    """zero-points u8 [G][N] -> device words [N][G8/8] (uint32), padded slots 0:
    group g of row n is nibble g % 8 of word g // 8 of the row."""
    z = np.asarray(zeros, dtype=np.uint32)
    G, N = z.shape
    G8 = padded_groups(G)
    full = np.zeros((N, G8), dtype=np.uint32)
    full[:, :G] = z.T
    nib = full.reshape(N, G8 // 8, 8)
    word = np.zeros((N, G8 // 8), dtype=np.uint32)
    for i in range(8):
        word |= nib[:, :, i] << np.uint32(4 * i)
    return word


def device_meta_bytes(N: int, K: int, group: int, fmt: str = "asym4"):
    """(scales, zeros) byte counts of the device metadata layout."""
    G8 = padded_groups(K // group)
    return 2 * G8 * N, G8 * N // 2 if fmt == "asym4" else 0


def quantize_and_pack(w, group: int, fmt: str = "asym4"):
    """Full offline step: (qweight bytes, device scales, device zero words or None,
    codes, scale bits, zeros)."""
    codes, s_bits, zeros = quantize_groupwise(w, group, fmt)
    zdev = pack_zeros_device(zeros, group) if fmt == "asym4" else None
    return (pack_device(codes, fmt), pack_scales_device(s_bits, group), zdev, codes, s_bits, zeros)


# ---------------------------------------------------------------------------
# The product. Activations stay 16-bit and the multiply is an ordinary
# floating-point one against the rebuilt weights ("Weight-Only Quantization
# Explained", "What W4A16 actually names" and "What it costs"). Here the
# accumulation is fp64 (exact products of fp16/bf16 and s*(q-z)).
# ---------------------------------------------------------------------------


def linear_ref(x_bits, x_dtype: str, w_hat):
    """y_ref [M][N] = x @ w_hat^T and A [M][N] = |x| @ |w_hat|^T, both fp64."""
    x = act_bits_to_f64(x_bits, x_dtype)
    if x.ndim == 1:
        x = x[None, :]
    w_hat = np.asarray(w_hat, dtype=np.float64)
    y = x @ w_hat.T
    a = np.abs(x) @ np.abs(w_hat).T
    return y, a


def linear_ref_rows(x_bits, x_dtype: str, codes, scale_bits, zeros, group: int, cols=None):
    """Same as linear_ref but dequantises only the requested output columns n."""
    codes = np.asarray(codes)
    if cols is not None:
        codes = codes[cols]
        scale_bits = np.asarray(scale_bits)[:, cols]
        zeros = np.asarray(zeros)[:, cols]
    w_hat = dequantize(codes, scale_bits, zeros, group)
    return linear_ref(x_bits, x_dtype, w_hat)


TOL_REL = 2e-3
TOL_ABS = 1e-5


def out_half_ulp(y64, dtype: str) -> np.ndarray:
    """Half the spacing of the output format (fp16: 11 significant bits, bf16:
    8) at |y|, subnormal range included: the largest error of rounding an exact
    value once, to nearest, into that format."""
    p, emin = (11, -14) if dtype == "f16" else (8, -126)
    mag = np.abs(np.asarray(y64, dtype=np.float64))
    _, ex = np.frexp(mag)                       # mag = f * 2**ex, f in [0.5, 1)
    e = np.where(mag > 0, np.maximum(ex - 1, emin), emin)
    return np.ldexp(1.0, (e - p).astype(np.int64))


def error_ratio(y_gpu, y_ref, a, out_dtype: str | None = None) -> np.ndarray:
    """|y - y_ref| / (2e-3 * sum|x*w_hat| + 1e-5 [+ half a bf16 ulp]); the
    acceptance bar is <= 1.

    The bar is the stated tolerance, 2e-3 of sum|x*w_hat| plus 1e-5. Every
    implementation rounds its result once to the output type (to nearest
    even). For fp16 outputs that rounding costs at most half an fp16 ulp,
    2**-11 of |y| (and 2**-25 absolute in the subnormal range), a quarter of
    the bar at worst since |y| <= sum|x*w_hat|, so fp16 is held to the bare
    bar. For bf16 it costs up to 2**-8 of |y|, more than 2e-3: a correctly
    rounded exact result could fail when |y| is close to sum|x*w_hat| (short
    K), so with out_dtype "bf16" half a bf16 ulp at |y| joins the budget."""
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    budget = TOL_REL * a + TOL_ABS
    if out_dtype == "bf16":
        budget = budget + out_half_ulp(np.maximum(np.abs(y_gpu), np.abs(y_ref)), out_dtype)
    return np.abs(y_gpu - y_ref) / budget


# ---------------------------------------------------------------------------
# Quantisation quality. The instagit comparison page ("Implementation
# Architecture": the error-analysis routine) reports four figures for a
# quantised tensor: mean squared error, signal-to-noise ratio in dB, cosine
# similarity and the largest error. Its formulas are not printed; these are the
# standard definitions, over the flattened matrix, in fp64:
#   MSE  = sum (w - w_hat)^2 / (N K)
#   SNR  = 10 log10( sum w^2 / sum (w - w_hat)^2 )      (+inf when exact)
#   cos  = sum w w_hat / sqrt(sum w^2 * sum w_hat^2)   (1 when both are zero)
#   max  = max |w - w_hat|
# ---------------------------------------------------------------------------


def quant_error_sums(w, w_hat):
    """(sum d^2, sum w^2, sum w_hat^2, sum w w_hat, max |d|) with d = w - w_hat, fp64."""
    w = np.asarray(w, dtype=np.float32).astype(np.float64)
    h = np.asarray(w_hat, dtype=np.float64)
    d = w - h
    return (float(np.sum(d * d)), float(np.sum(w * w)), float(np.sum(h * h)), float(np.sum(w * h)),
            float(np.max(np.abs(d), initial=0.0)))


def quant_error_stats(sums, count: int):
    """(MSE, SNR dB, cosine, max error) from the five sums over `count` weights."""
    d2, w2, h2, wh, mx = sums
    mse = d2 / count
    snr = np.inf if d2 == 0.0 else (10.0 * np.log10(w2 / d2) if w2 > 0.0 else -np.inf)
    if w2 == 0.0 and h2 == 0.0:
        cos = 1.0
    elif w2 == 0.0 or h2 == 0.0:
        cos = 0.0
    else:
        cos = wh / np.sqrt(w2 * h2)
    return mse, float(snr), float(cos), mx


def quant_error(w, codes, scale_bits, zeros, group: int):
    """Quality report of one quantised matrix: (MSE, SNR dB, cosine, max error)."""
    w_hat = dequantize(codes, scale_bits, zeros, group)
    return quant_error_stats(quant_error_sums(w, w_hat), w_hat.size)


# ---------------------------------------------------------------------------
# AWQ, the deployable half. Salient input channels are scaled up before
# quantisation and the activations are scaled down to compensate (instagit
# comparison page, "AWQ: Activation-Aware Weight Quantization"; "Weight-Only
# Quantisation": deployment stays ordinary groupwise INT4). The choice of the
# factors needs calibration activations and is not part of this library; the
# factors a_k > 0 are an input. Offline: w'[n][k] = w[n][k] * a_k (fp32), then
# the usual quantiser. At run time the activations are multiplied by
# m_k = 1 / a_k, given as fp32: x'[m][k] = rne16(fp32(x[m][k] * m_k)), one
# fp32 product rounded once to the activation type, and y = x' w_hat'^T.
# ---------------------------------------------------------------------------


def awq_fold_weights(w, a):
    """w' = w * a along K (fp32 product): the weights AWQ quantises."""
    return (np.asarray(w, dtype=np.float32) * np.asarray(a, dtype=np.float32)[None, :]).astype(np.float32)


def awq_scale_activations(x_bits, dtype: str, act_mul):
    """x' bits = rne16(fp32(x * m)) for 16-bit activation bits x [M][K] and fp32 m [K]."""
    x = act_bits_to_f64(x_bits, dtype).astype(np.float32)       # exact widening
    prod = x * np.asarray(act_mul, dtype=np.float32)[None, :]     # IEEE fp32 product
    return f32_to_f16_bits(prod) if dtype == "f16" else f32_to_bf16_bits(prod)


# ---------------------------------------------------------------------------
# K-quant-style super-blocks (kq4). "Quantization Is Not a Zip File", "How to
# read common GGUF quantization names": K-quants keep sub-block scales and
# minima inside 256-weight super-blocks. The pages give no more than that;
# the reading used here (listed in the design notes) takes the asymmetric
# quantiser above per 32-weight sub-block and quantises its scale and minimum
# a second time, against the super-block's largest:
#   per sub-block j:  lo = min(0, min w), hi = max(0, max w),
#                     s_j = (hi - lo) / 15,  mn_j = 0 - lo       (fp32; +0, never -0)
#   per super-block:  d = fp16(max_j s_j / 63), dmin = fp16(max_j mn_j / 63)
#                     (0 -> 2**-24)
#   sc_j = clamp(rint(s_j / d), 0, 63), mq_j = clamp(rint(mn_j / dmin), 0, 63)
#   S_j = d * sc_j, M_j = dmin * mq_j                             (fp32, exact)
#   q = clamp(rint((w + M_j) / S_j), 0, 15), and q = 0 where S_j = 0
#   w_hat = S_j * q - M_j
# Stored per (super-block u, output column n): a 16-byte record of four
# little-endian words {d | dmin << 16, sc bits 0-31, sc bits 32-47 | mq bits
# 0-15 << 16, mq bits 16-47}, where sc and mq are 48-bit fields holding the
# eight 6-bit values at bits 6j..6j+5; canonical records in [U][N] order
# (U = K / 256); the device keeps each row's records together, [N][U].
# 4 + 128/256 = 4.5 bits per weight.
# ---------------------------------------------------------------------------

KQ_SUPER = 256
KQ_SUB = 32
KQ_RECORD_BYTES = 16


def quantize_kquant(w):
    """fp32 w [N][K] (K % 256 == 0) -> (codes u8 [N][K], d bits u16 [U][N],
    dmin bits u16 [U][N], sc u8 [U][8][N], mq u8 [U][8][N])."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    if K % KQ_SUPER != 0 or K == 0:
        raise ValueError("K must be a positive multiple of 256")
    if not np.all(np.isfinite(w)) or np.max(np.abs(w), initial=0.0) >= 2.0 ** 18:
        raise ValueError("weights must be finite with |w| < 2**18")
    U = K // KQ_SUPER
    wb = w.reshape(N, U, KQ_SUPER // KQ_SUB, KQ_SUB)
    zero = np.float32(0.0)
    lo = np.minimum(wb.min(axis=3), zero)                       # [N][U][8]
    hi = np.maximum(wb.max(axis=3), zero)
    s = (hi - lo) / np.float32(15.0)
    mn = zero - lo                                               # +0 for a group without negatives
    d_bits = f32_to_f16_bits(s.max(axis=2) / np.float32(63.0))
    d_bits = np.where(d_bits == 0, F16_MIN_SUBNORMAL_BITS, d_bits).astype(np.uint16)
    m_bits = f32_to_f16_bits(mn.max(axis=2) / np.float32(63.0))
    m_bits = np.where(m_bits == 0, F16_MIN_SUBNORMAL_BITS, m_bits).astype(np.uint16)
    d = f16_bits_to_f32(d_bits)[:, :, None]
    dmin = f16_bits_to_f32(m_bits)[:, :, None]
    sc = np.clip(np.rint(s / d), 0, 63).astype(np.int32)
    mq = np.clip(np.rint(mn / dmin), 0, 63).astype(np.int32)
    S = d * sc.astype(np.float32)
    Mn = dmin * mq.astype(np.float32)
    num = wb + Mn[..., None]
    den = np.broadcast_to(S[..., None], num.shape)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(den > 0, np.rint(np.divide(num, den, where=den > 0, out=np.zeros_like(num))), 0.0)
    q = np.clip(r, 0, 15).astype(np.uint8)
    return (q.reshape(N, K), np.ascontiguousarray(d_bits.T), np.ascontiguousarray(m_bits.T),
            np.ascontiguousarray(sc.transpose(1, 2, 0).astype(np.uint8)),
            np.ascontiguousarray(mq.transpose(1, 2, 0).astype(np.uint8)))


def kquant_sub_params(d_bits, m_bits, sc, mq):
    """(S, M) fp64 [N][K/32]: the effective scale and minimum of every sub-block."""
    d = f16_bits_to_f64(d_bits).T                                # [N][U]
    dmin = f16_bits_to_f64(m_bits).T
    S = d[:, :, None] * np.asarray(sc, dtype=np.float64).transpose(2, 0, 1)
    M = dmin[:, :, None] * np.asarray(mq, dtype=np.float64).transpose(2, 0, 1)
    N = S.shape[0]
    return S.reshape(N, -1), M.reshape(N, -1)


def dequantize_kquant(codes, d_bits, m_bits, sc, mq) -> np.ndarray:
    """w_hat [N][K] = S_j * q - M_j in fp64."""
    codes = np.asarray(codes, dtype=np.uint8)
    N, K = codes.shape
    S, M = kquant_sub_params(d_bits, m_bits, sc, mq)
    q = codes.reshape(N, K // KQ_SUB, KQ_SUB).astype(np.float64)
    return (q * S[:, :, None] - M[:, :, None]).reshape(N, K)


def pack_kquant_device(d_bits, m_bits, sc, mq) -> np.ndarray:
    """Super-block records in device order, uint32 [N][U][4] (one row's records
    contiguous along K)."""
    return np.ascontiguousarray(pack_kquant_records(d_bits, m_bits, sc, mq).transpose(1, 0, 2))


def pack_kquant_records(d_bits, m_bits, sc, mq) -> np.ndarray:
    """Super-block records, uint32 [U][N][4] (layout above)."""
    d_bits = np.asarray(d_bits, dtype=np.uint64)
    U, N = d_bits.shape
    sc = np.asarray(sc, dtype=np.uint64)
    mq = np.asarray(mq, dtype=np.uint64)
    scf = np.zeros((U, N), dtype=np.uint64)
    mqf = np.zeros((U, N), dtype=np.uint64)
    for j in range(KQ_SUPER // KQ_SUB):
        scf |= sc[:, j, :] << np.uint64(6 * j)
        mqf |= mq[:, j, :] << np.uint64(6 * j)
    rec = np.zeros((U, N, 4), dtype=np.uint64)
    rec[:, :, 0] = d_bits | (np.asarray(m_bits, dtype=np.uint64) << np.uint64(16))
    rec[:, :, 1] = scf & np.uint64(0xFFFFFFFF)
    rec[:, :, 2] = (scf >> np.uint64(32)) | ((mqf & np.uint64(0xFFFF)) << np.uint64(16))
    rec[:, :, 3] = mqf >> np.uint64(16)
    return rec.astype(np.uint32)
