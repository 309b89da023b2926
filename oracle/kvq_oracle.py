"""Plain, slow, obviously-correct CPU oracle of the quantized session KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module; only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` do.  It shares no code with the HIP
library (no kernels, headers, helpers, tables or constants).

What it computes, and where the pages say so
--------------------------------------------
* Different bit widths for keys and values (FP16, K8V8, K8V4, K4V8, K4V4):
  "KVSplit -- contexto 2 a 3 vezes mais longo em Apple Silicon"
  (pt.news.hada.io, topic 20969), sections "Principais resultados de
  benchmark" and "Assimetria entre key e value"; the int8/int4 split also in
  "KVBoost acelera inferencia de LLMs em 4,49x com cache reutilizavel",
  section "Impacto".
* The block format (32 elements + one fp16 scale, i.e. 8.5 and 4.5 bits per
  element) is not stated on the pages; it is the reading that reproduces every
  footprint the KVSplit page prints (section "Uso de memoria conforme o
  comprimento da sequencia").  The 256-token capacity granule is the reading of
  the same page's remark on 256-byte page alignment (section "Otimizacao para
  Apple Silicon e limitacoes"), which is what makes its 128-token row come out.
* Quantize on append, independent of the model weights: KVSplit page,
  section "Opinioes no Hacker News" (the cache is quantized at run time as
  tokens are processed).
* Keep the cache between turns and process only the new tokens:
  "Reutilizacao de Cache KV para Conversas Longas no Apple Silicon Oferece
  Aceleracao de 200x" (openclawradar.com), section "Principais Descobertas e
  Benchmarks".
* Attention itself is the plain definition softmax(sigma * q.K^T) V, in fp64,
  over the dequantized cache.
* The same attention in two passes (per-range partial softmax sums over disjoint
  key ranges, then their log-sum-exp merge) is the exact identity the split
  kernels rely on; the pages do not discuss splitting.

Conventions fixed here (readings where the pages are silent; each is listed
in the design notes of the repository):
  per (token, KV head, 32 consecutive elements along head_dim):
    amax = max |x_i|                       (x widened exactly to fp32)
    d    = fp16_RNE(min(fp32(amax / qmax), 65504)),  qmax = 127 or 7
    q_i  = 0 if d == 0 else clamp(RHAZ(fp32(x_i / d)), -qmax, qmax)
  8-bit codes are stored as two's-complement int8; 4-bit codes as the nibble
  u = q + 8, byte j of a block holding u[2j] in the low and u[2j+1] in the
  high nibble; d is stored as little-endian fp16 bits.  The FP16 layout stores
  fp16_RNE(x) and has no scale plane.
  Planes are kept per (layer, KV head): Kc[cap][code bytes], Ks[cap][scale
  bytes], Vc, Vs, token-major.  cap = round_up(max_tokens, 256).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "LAYOUTS", "LAYOUT_IDS", "BLOCK", "GRANULE", "layout_bits", "code_row_bytes",
    "scale_row_bytes", "capacity", "layout_footprint_bytes", "f32_to_f16",
    "block_scale", "rhaz", "quantize_rows", "pack_codes", "unpack_codes",
    "pack_scales", "unpack_scales", "encode_rows", "dequant_rows", "OracleCache", "OracleLayeredCache",
    "E4M3_MAX", "e4m3_values", "e4m3_encode", "mx_scale_exponent", "mx_quantize_rows", "mx_dequant_rows",
    "attend_decode", "attend_chunk", "attention_exact", "to_f32",
    "split_partial", "merge_partials", "decode_partials", "chunk_partials", "LOG2E",
]

#: layout id -> (name, key bits, value bits).  16 means the fp16 control.
LAYOUTS = {0: ("FP16", 16, 16), 1: ("K8V8", 8, 8), 2: ("K8V4", 8, 4),
           3: ("K4V8", 4, 8), 4: ("K4V4", 4, 4), 5: ("KF8V4", "f8", 4)}
LAYOUT_IDS = {v[0]: k for k, v in LAYOUTS.items()}
BLOCK = 32          # elements per quantization block (reading; see module doc)
GRANULE = 256       # capacity granule in tokens (reading; see module doc)
FP16_MAX = 65504.0


def layout_bits(layout: int) -> tuple[int, int]:
    """(key bits, value bits) of a layout id."""
    _, kb, vb = LAYOUTS[int(layout)]
    return kb, vb


def code_row_bytes(bits, head_dim: int) -> int:
    """Bytes of codes per (token, KV head): 2D for fp16, D for 8-bit and fp8, D/2 for 4-bit."""
    return {16: 2 * head_dim, 8: head_dim, "f8": head_dim, 4: head_dim // 2}[bits]


def scale_row_bytes(bits, head_dim: int) -> int:
    """Bytes of scales per (token, KV head), one per 32-element block: fp16 (2 bytes) for
    8/4-bit codes, a power-of-two exponent byte for fp8 codes; none for fp16."""
    if bits == 16:
        return 0
    return (1 if bits == "f8" else 2) * (head_dim // BLOCK)


def capacity(max_tokens: int) -> int:
    """Tokens allocated per (layer, KV head): max_tokens rounded up to 256."""
    return -(-int(max_tokens) // GRANULE) * GRANULE


def layout_footprint_bytes(layout: int, n_layers: int, n_kv_heads: int,
                           head_dim: int, max_tokens: int) -> int:
    """Bytes of all planes: L * Hkv * cap * (K row + V row), rows including scales."""
    kb, vb = layout_bits(layout)
    per_token = (code_row_bytes(kb, head_dim) + scale_row_bytes(kb, head_dim)
                 + code_row_bytes(vb, head_dim) + scale_row_bytes(vb, head_dim))
    return n_layers * n_kv_heads * capacity(max_tokens) * per_token


# --------------------------------------------------------------------------
# scalar conventions
# --------------------------------------------------------------------------
def to_f32(x) -> np.ndarray:
    """Widen inputs to fp32.  bf16 and fp16 values widen exactly; callers hand
    bf16 data in as fp32 arrays that hold bf16-representable values."""
    return np.asarray(x, dtype=np.float32)


def f32_to_f16(x32: np.ndarray) -> np.ndarray:
    """IEEE round-to-nearest-even fp32 -> fp16 (numpy's cast)."""
    return np.asarray(x32, dtype=np.float32).astype(np.float16)


def block_scale(amax32: np.ndarray, qmax: int) -> np.ndarray:
    """d = fp16_RNE(fp32(amax / qmax)), saturated at the largest finite fp16."""
    d32 = np.asarray(amax32, dtype=np.float32) / np.float32(qmax)   # IEEE fp32 division
    d32 = np.minimum(d32, np.float32(FP16_MAX))
    return f32_to_f16(d32)


def rhaz(y32: np.ndarray) -> np.ndarray:
    """Round half away from zero, evaluated in fp64 (exact for fp32 inputs)."""
    y = np.asarray(y32, dtype=np.float64)
    return np.sign(y) * np.floor(np.abs(y) + 0.5)


# --------------------------------------------------------------------------
# codec
# --------------------------------------------------------------------------
def quantize_rows(x, bits: int):
    """Quantize rows [n, D] block by block.

    Returns (codes int16 [n, D], scales float16 [n, D/32]) for 8/4 bits, or
    (fp16 values [n, D], None) for the fp16 control.
    """
    x32 = to_f32(x)
    n, dim = x32.shape
    if bits == 16:
        return f32_to_f16(x32), None
    qmax = {8: 127, 4: 7}[bits]
    xb = x32.reshape(n, dim // BLOCK, BLOCK)
    amax = np.max(np.abs(xb), axis=2)
    d16 = block_scale(amax, qmax)
    d32 = d16.astype(np.float32)[:, :, None]
    y = np.zeros_like(xb)
    np.divide(xb, d32, out=y, where=(d32 != 0))                      # fp32 division
    q = np.clip(rhaz(y), -qmax, qmax)
    q = np.where(d32 != 0, q, 0.0)
    return q.astype(np.int16).reshape(n, dim), d16


def pack_codes(codes, bits: int) -> np.ndarray:
    """Codes [n, D] -> bytes [n, code_row_bytes]."""
    if bits == 16:
        c = np.ascontiguousarray(np.asarray(codes, dtype=np.float16))
        return c.view(np.uint8).reshape(c.shape[0], -1)
    c = np.asarray(codes, dtype=np.int16)
    if bits == 8:
        return c.astype(np.int8).view(np.uint8)
    u = (c + 8).astype(np.uint8)                                     # nibble in [1, 15]
    return (u[:, 0::2] | (u[:, 1::2] << 4)).astype(np.uint8)


def unpack_codes(packed, bits: int, head_dim: int) -> np.ndarray:
    """Inverse of pack_codes.  Returns int16 codes, or float16 for the control."""
    p = np.asarray(packed, dtype=np.uint8)
    if bits == 16:
        return np.ascontiguousarray(p).view(np.float16).reshape(p.shape[0], head_dim)
    if bits == 8:
        return p.view(np.int8).astype(np.int16)
    out = np.empty((p.shape[0], head_dim), dtype=np.int16)
    out[:, 0::2] = (p & 0x0F).astype(np.int16) - 8
    out[:, 1::2] = (p >> 4).astype(np.int16) - 8
    return out


def pack_scales(d16) -> np.ndarray:
    """fp16 scales [n, nb] -> little-endian bytes [n, 2 nb]."""
    d = np.ascontiguousarray(np.asarray(d16, dtype="<f2"))
    return d.view(np.uint8).reshape(d.shape[0], -1)


def unpack_scales(packed) -> np.ndarray:
    p = np.ascontiguousarray(np.asarray(packed, dtype=np.uint8))
    return p.view("<f2").reshape(p.shape[0], -1)


def encode_rows(x, bits):
    """Rows [n, D] -> (code bytes [n, cb], scale bytes [n, sb] or None)."""
    if bits == "f8":
        return mx_quantize_rows(x)
    codes, d16 = quantize_rows(x, bits)
    return pack_codes(codes, bits), (None if d16 is None else pack_scales(d16))


def dequant_rows(code_bytes, scale_bytes, bits, head_dim: int) -> np.ndarray:
    """x_hat = q * d per element (exact in fp64), or the fp16 value for the control."""
    if bits == "f8":
        return mx_dequant_rows(code_bytes, scale_bytes)
    c = unpack_codes(code_bytes, bits, head_dim)
    if bits == 16:
        return c.astype(np.float64)
    d = unpack_scales(scale_bytes).astype(np.float64)
    return c.astype(np.float64) * np.repeat(d, BLOCK, axis=1)


# --------------------------------------------------------------------------
# fp8 keys: OCP MX "MXFP8" blocks (reading of the offloading page's FP8 alternative,
# "KV Cache Offloading for Context-Intensive Tasks", section on quantization)
# --------------------------------------------------------------------------
# Each 32-element block stores one shared power-of-two scale X = 2^e as a biased exponent
# byte (e + 127) and 32 elements y = x / X as OCP FP8 E4M3 codes: sign, 4 exponent bits
# (bias 7), 3 mantissa bits, subnormals, no infinities, S.1111.111 = NaN, largest 448.
# e = floor(log2(amax)) - 8 (8 = the largest E4M3 exponent), clamped to [-127, 127]
# (e = -127 for an all-zero block); elements round to nearest, ties to even, saturate at
# +-448, and a result of zero is stored as +0.
E4M3_MAX = 448.0


def e4m3_values() -> np.ndarray:
    """The value of each of the 256 E4M3 codes (NaN for 0x7F and 0xFF)."""
    v = np.empty(256, np.float64)
    for c in range(256):
        sign = -1.0 if c & 0x80 else 1.0
        e, m = (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            v[c] = np.nan
        elif e == 0:
            v[c] = sign * m * 2.0 ** -9
        else:
            v[c] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return v


def e4m3_encode(y) -> np.ndarray:
    """E4M3 codes of exact values y (fp64): round to nearest, ties to even, saturate."""
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    code = np.zeros(y.shape, np.int64)
    sat = a >= E4M3_MAX
    sub = a < 2.0 ** -6
    norm = ~sat & ~sub
    code[sat] = 0x7E
    code[sub] = np.rint(a[sub] * 2.0 ** 9).astype(np.int64)          # 8 lands on 2^-6 = 0x08
    _, k = np.frexp(a[norm])
    e = k.astype(np.int64) - 1                                        # floor(log2 a), -6..8
    m = np.rint(a[norm] * np.exp2(3.0 - e)).astype(np.int64)           # 8..16
    up = m == 16
    e[up] += 1
    m[up] = 8
    code[norm] = ((e + 7) << 3) | (m - 8)
    code[norm & (code == 0x7F)] = 0x7E
    code[(y < 0) & (code != 0)] |= 0x80
    return code.astype(np.uint8)


def mx_scale_exponent(amax32) -> np.ndarray:
    """e of X = 2^e for block maxima amax (fp32): floor(log2 amax) - 8 in [-127, 127]."""
    a = np.asarray(amax32, dtype=np.float64)
    _, k = np.frexp(a)
    e = np.where(a > 0, k.astype(np.int64) - 1 - 8, -127)
    return np.clip(e, -127, 127)


def mx_quantize_rows(x):
    """Rows [n, D] -> (E4M3 code bytes [n, D], scale exponent bytes [n, D/32])."""
    x32 = to_f32(x)
    n, dim = x32.shape
    xb = x32.reshape(n, dim // BLOCK, BLOCK).astype(np.float64)
    e = mx_scale_exponent(np.max(np.abs(xb), axis=2).astype(np.float32))
    codes = e4m3_encode(xb * np.exp2(-e.astype(np.float64))[:, :, None])
    return codes.reshape(n, dim), (e + 127).astype(np.uint8)


def mx_dequant_rows(code_bytes, scale_bytes) -> np.ndarray:
    """x_hat = E4M3 value * 2^(scale byte - 127), exact in fp64."""
    c = np.asarray(code_bytes, dtype=np.uint8)
    e = np.asarray(scale_bytes, dtype=np.uint8).astype(np.float64) - 127.0
    return e4m3_values()[c] * np.repeat(np.exp2(e), BLOCK, axis=1)


# --------------------------------------------------------------------------
# the session cache
# --------------------------------------------------------------------------
class OracleCache:
    """Planes per (layer, KV head), appended token by token in order."""

    def __init__(self, layout: int, n_layers: int, n_kv_heads: int, head_dim: int,
                 max_tokens: int):
        if head_dim % BLOCK:
            raise ValueError("head_dim must be a multiple of 32")
        self.layout, self.L, self.Hkv, self.D = int(layout), n_layers, n_kv_heads, head_dim
        self.max_tokens = int(max_tokens)
        self.cap = capacity(max_tokens)
        self.kbits, self.vbits = layout_bits(layout)
        self.len = [0] * n_layers
        shp = (n_layers, n_kv_heads, self.cap)
        self.Kc = np.zeros(shp + (code_row_bytes(self.kbits, head_dim),), np.uint8)
        self.Ks = np.zeros(shp + (scale_row_bytes(self.kbits, head_dim),), np.uint8)
        self.Vc = np.zeros(shp + (code_row_bytes(self.vbits, head_dim),), np.uint8)
        self.Vs = np.zeros(shp + (scale_row_bytes(self.vbits, head_dim),), np.uint8)

    def footprint_bytes(self) -> int:
        return self.Kc.nbytes + self.Ks.nbytes + self.Vc.nbytes + self.Vs.nbytes

    def append(self, layer: int, k, v) -> None:
        """Quantize and store new tokens K, V [n, Hkv, D] at rows [len, len + n)."""
        k32, v32 = to_f32(k), to_f32(v)
        n = k32.shape[0]
        t0 = self.len[layer]
        if t0 + n > self.max_tokens:
            raise ValueError("append past max_tokens")
        for h in range(self.Hkv):
            kc, ks = encode_rows(k32[:, h, :], self.kbits)
            vc, vs = encode_rows(v32[:, h, :], self.vbits)
            self.Kc[layer, h, t0:t0 + n] = kc
            self.Vc[layer, h, t0:t0 + n] = vc
            if ks is not None:
                self.Ks[layer, h, t0:t0 + n] = ks
            if vs is not None:
                self.Vs[layer, h, t0:t0 + n] = vs
        self.len[layer] = t0 + n

    def reset(self) -> None:
        self.len = [0] * self.L

    def keys(self, layer: int, kv_head: int, t1: int | None = None) -> np.ndarray:
        """Dequantized keys [t1, D] in fp64 (t1 defaults to the cached length)."""
        t1 = self.len[layer] if t1 is None else t1
        return dequant_rows(self.Kc[layer, kv_head, :t1], self.Ks[layer, kv_head, :t1],
                            self.kbits, self.D)

    def values(self, layer: int, kv_head: int, t1: int | None = None) -> np.ndarray:
        t1 = self.len[layer] if t1 is None else t1
        return dequant_rows(self.Vc[layer, kv_head, :t1], self.Vs[layer, kv_head, :t1],
                            self.vbits, self.D)


class OracleLayeredCache:
    """A cache whose layer l stores its keys and values in layouts[l] (layer-specific
    quantization, planned on the KVSplit page, section "Configuracao recomendada e
    roadmap"): one single-layer OracleCache per layer, with the same interface."""

    def __init__(self, layouts, n_kv_heads: int, head_dim: int, max_tokens: int):
        self.layouts = [int(x) for x in layouts]
        self.layers = [OracleCache(lay, 1, n_kv_heads, head_dim, max_tokens) for lay in self.layouts]
        self.L, self.Hkv, self.D = len(self.layouts), n_kv_heads, head_dim
        self.max_tokens, self.cap = int(max_tokens), capacity(max_tokens)

    @property
    def len(self):
        return [c.len[0] for c in self.layers]

    def footprint_bytes(self) -> int:
        return sum(c.footprint_bytes() for c in self.layers)

    def append(self, layer: int, k, v) -> None:
        self.layers[layer].append(0, k, v)

    def reset(self) -> None:
        for c in self.layers:
            c.reset()

    def plane(self, layer: int, name: str) -> np.ndarray:
        """Plane `name` (Kc, Ks, Vc, Vs) of one layer: [Hkv, cap, row bytes]."""
        return getattr(self.layers[layer], name)[0]

    def keys(self, layer: int, kv_head: int, t1: int | None = None) -> np.ndarray:
        return self.layers[layer].keys(0, kv_head, t1)

    def values(self, layer: int, kv_head: int, t1: int | None = None) -> np.ndarray:
        return self.layers[layer].values(0, kv_head, t1)


# --------------------------------------------------------------------------
# attention over the dequantized cache (fp64)
# --------------------------------------------------------------------------
def attention_exact(q, keys, values, sm_scale: float) -> np.ndarray:
    """softmax(sm_scale * q K^T) V for query rows q [r, D] against keys/values [T, D], fp64."""
    q64 = np.asarray(q, dtype=np.float64)
    s = sm_scale * (q64 @ np.asarray(keys, dtype=np.float64).T)
    s -= s.max(axis=1, keepdims=True)
    w = np.exp(s)
    return (w @ np.asarray(values, dtype=np.float64)) / w.sum(axis=1, keepdims=True)


def attend_decode(caches, layer: int, q, sm_scale: float) -> np.ndarray:
    """One query per session: q [S, Hq, D] against each session's whole cached length.

    q head h reads KV head h // (Hq / Hkv) (contiguous GQA groups).
    """
    q = to_f32(q)
    n_s, hq, dim = q.shape
    out = np.zeros((n_s, hq, dim), np.float64)
    for s, c in enumerate(caches):
        if c.len[layer] == 0:
            raise ValueError("decode on an empty cache")
        g = hq // c.Hkv
        for h in range(c.Hkv):
            out[s, h * g:(h + 1) * g] = attention_exact(
                q[s, h * g:(h + 1) * g], c.keys(layer, h), c.values(layer, h), sm_scale)
    return out


def attend_chunk(cache: OracleCache, layer: int, q, n_new: int, sm_scale: float,
                 rows=None, row_block: int = 64) -> np.ndarray:
    """Causal attention of the last n_new cached positions.

    q [n_new, Hq, D]; query j sits at absolute position len - n_new + j and sees
    keys [0, that position] (inclusive), its own chunk read back from the
    quantized cache.  ``rows`` restricts the computation to those query indices
    (output [len(rows), Hq, D]); ``row_block`` only bounds memory.
    """
    q = to_f32(q)
    total = cache.len[layer]
    if not 0 < n_new <= total:
        raise ValueError("chunk must already be appended")
    rows = np.arange(n_new) if rows is None else np.asarray(rows)
    hq, dim = q.shape[1], q.shape[2]
    g = hq // cache.Hkv
    out = np.zeros((len(rows), hq, dim), np.float64)
    for h in range(cache.Hkv):
        kh, vh = cache.keys(layer, h, total), cache.values(layer, h, total)
        for b0 in range(0, len(rows), row_block):
            rb = rows[b0:b0 + row_block]
            pos = total - n_new + rb                                   # absolute positions
            qb = q[rb, h * g:(h + 1) * g, :].astype(np.float64).reshape(-1, dim)
            s = sm_scale * (qb @ kh.T)                                  # [r*g, total]
            visible = np.arange(total)[None, :] <= np.repeat(pos, g)[:, None]
            s[~visible] = -np.inf
            s -= s.max(axis=1, keepdims=True)
            w = np.exp(s)
            o = (w @ vh) / w.sum(axis=1, keepdims=True)
            out[b0:b0 + len(rb), h * g:(h + 1) * g] = o.reshape(len(rb), g, dim)
    return out


# --------------------------------------------------------------------------
# attention in two passes: per-split partial sums and their merge (fp64)
# --------------------------------------------------------------------------
# Splitting the keys into disjoint ranges and recombining the per-range softmax sums
# is exact: with x_t the score of key t in base-2 units, sum_t 2^x_t v_t and
# sum_t 2^x_t are sums over the ranges, each kept relative to its own reference m.
# The pages do not discuss it; it is how a long context is spread over workgroups
# (or devices), and the library exposes both passes.
LOG2E = 1.4426950408889634


def split_partial(q, keys, values, sm_scale: float):
    """(o, m, l) of query rows q [r, D] over one key range keys/values [n, D].

    x_t = sm_scale * log2(e) * q . k_t;  m = max_t x_t;  l = sum_t 2^(x_t - m);
    o = sum_t 2^(x_t - m) v_t.  An empty range gives m = -inf, l = 0, o = 0.
    """
    q64 = np.asarray(q, dtype=np.float64)
    r, dim = q64.shape
    keys = np.asarray(keys, dtype=np.float64)
    if keys.shape[0] == 0:
        return np.zeros((r, dim)), np.full(r, -np.inf), np.zeros(r)
    x = (sm_scale * LOG2E) * (q64 @ keys.T)
    m = x.max(axis=1)
    w = np.exp2(x - m[:, None])
    return w @ np.asarray(values, dtype=np.float64), m, w.sum(axis=1)


def merge_partials(o, m, l):
    """Normalized output from split partials o [.., S, D], m [.., S], l [.., S]:
    M = max_s m_s, o = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s; splits with
    m = -inf (no key) weigh nothing."""
    o, m, l = (np.asarray(a, dtype=np.float64) for a in (o, m, l))
    big = m.max(axis=-1, keepdims=True)
    w = np.where(np.isneginf(m), 0.0, np.exp2(m - np.where(np.isneginf(big), 0.0, big)))
    return (w[..., None] * o).sum(axis=-2) / (w * l).sum(axis=-1)[..., None]


def decode_partials(caches, layer: int, q, sm_scale: float, n_splits: int, per_split: int):
    """Per session, q head and split s (tokens [s * per_split, min((s + 1) * per_split, len))):
    (o [S, Hq, n_splits, D], m [S, Hq, n_splits], l [S, Hq, n_splits])."""
    q = to_f32(q)
    n_s, hq, dim = q.shape
    o = np.zeros((n_s, hq, n_splits, dim))
    m = np.full((n_s, hq, n_splits), -np.inf)
    l = np.zeros((n_s, hq, n_splits))
    for b, c in enumerate(caches):
        g = hq // c.Hkv
        total = c.len[layer]
        for h in range(c.Hkv):
            kh, vh = c.keys(layer, h), c.values(layer, h)
            for sp in range(n_splits):
                a, e = min(sp * per_split, total), min((sp + 1) * per_split, total)
                o[b, h * g:(h + 1) * g, sp], m[b, h * g:(h + 1) * g, sp], l[b, h * g:(h + 1) * g, sp] = \
                    split_partial(q[b, h * g:(h + 1) * g], kh[a:e], vh[a:e], sm_scale)
    return o, m, l


def chunk_partials(cache: OracleCache, layer: int, q, n_new: int, sm_scale: float, n_splits: int,
                   per_split: int, rows=None):
    """Per new token j (position len - n_new + j), q head and split s: the partials over the
    keys of [s * per_split, (s + 1) * per_split) that j sees (t <= its position).
    ``rows`` restricts the computation to those tokens.  Shapes as decode_partials with
    the token index first."""
    q = to_f32(q)
    total = cache.len[layer]
    if not 0 < n_new <= total:
        raise ValueError("chunk must already be appended")
    rows = np.arange(n_new) if rows is None else np.asarray(rows)
    hq, dim = q.shape[1], q.shape[2]
    g = hq // cache.Hkv
    o = np.zeros((len(rows), hq, n_splits, dim))
    m = np.full((len(rows), hq, n_splits), -np.inf)
    l = np.zeros((len(rows), hq, n_splits))
    for h in range(cache.Hkv):
        kh, vh = cache.keys(layer, h, total), cache.values(layer, h, total)
        for i, j in enumerate(rows):
            end = total - n_new + int(j) + 1                    # keys [0, end) are visible
            for sp in range(n_splits):
                a, e = min(sp * per_split, end), min((sp + 1) * per_split, end)
                o[i, h * g:(h + 1) * g, sp], m[i, h * g:(h + 1) * g, sp], l[i, h * g:(h + 1) * g, sp] = \
                    split_partial(q[j, h * g:(h + 1) * g], kh[a:e], vh[a:e], sm_scale)
    return o, m, l
