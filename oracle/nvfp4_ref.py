"""CPU reference (oracle) for attention over a paged NVFP4 KV cache.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  The library never calls it and shares
no code with it.

Plain numpy, float64, written for readability rather than speed.  Sources:

  [PF]  page "Re-enable split-KV for NVFP4 KV cache in prefill path"
        (jethac/flashinfer pull request 1; a series of commit messages)
  [XQA] page "Support NVFP4 KV cache decode on SM120"
        (flashinfer-ai/flashinfer pull request 2520)
  [FIX] page "fix(attention): correct SM120 NVFP4 qk_correction layout, row-sum
        reduction, and lse" (flashinfer-ai/flashinfer pull request 3838)

The pages name the formats (packed uint8 holding two e2m1 values per byte, one
FP8 e4m3 scale per 16 head-dim elements of one token and head) but do not spell
out the bit layouts, nibble order or rounding.  The readings taken here:

  * e2m1: sign bit 3, magnitude codes 0..7 = 0, 0.5, 1, 1.5, 2, 3, 4, 6 (OCP MX).
  * e4m3fn: 1 sign, 4 exponent bits (bias 7), 3 mantissa bits, subnormals,
    largest finite 448, 0x7F / 0xFF are NaN, no infinities (OCP FP8).
  * block scale s = RNE_e4m3(amax / (6 g)), saturating at 448; element code
    = RNE_e2m1(|x| / (s g)) with ties to the even code, saturating at 6, and the
    sign bit copied from x (so -0 and small negatives give nibble 0x8).  When
    s == 0 every magnitude code is 0.
  * byte j of a row holds element 2j in its low nibble and 2j+1 in its high one.
  * dequantised value = e2m1 * s * g, where g is the per-tensor global scale.
  * kv head of qo head h is h // (Hq / Hkv).
  * causal mask is aligned to the bottom right: query row i of a request with
    q_b rows and L_b keys sees keys j <= i + (L_b - q_b).
  * LSE is the natural-log sum of exp of the scaled scores; a row that sees no
    key gets O = 0 and LSE = -inf.
  * FP8 KV (the 1-byte KV type the pages run beside NVFP4): one e4m3fn byte per
    element, code = sign | RNE_e4m3(|x| / g) saturating at 448, value = e4m3 * g.
  * Ragged (non-paged) KV: request b's rows are rows kv_indptr[b] .. kv_indptr[b+1]-1
    of one [rows, H, W] array.
  * Packed custom masks: request b's mask is a [q_b, L_b] boolean array, row-major,
    1 = visible; each request's bits are packed on their own (little-endian bits within
    a byte, padded to a whole byte), so its bits start at byte sum of ceil(q_b' L_b' / 8)
    over the requests before it; a custom mask replaces the causal rule.
  * Rotary position embedding (in-kernel RoPE): the pages give no formula.  Reading:
    the rotary embedding of RoFormer in its rotate-half arrangement, where element i
    and element i + Dk/2 of a Q or K row form a pair rotated by pos * w_i, with
    w_i = theta^(-2i/Dk) / scale for i < Dk/2 (theta 1e4 by default; scale > 1
    stretches positions linearly).  Half the QK head dim of frequencies, as the pages'
    frequency table holds, spanning Dk also when Dv is smaller.  Key j of a request
    sits at position j (the cache holds un-rotated keys); query row i of a request
    with q_b rows and L_b keys at L_b - q_b + i, the causal rule's alignment.
"""
from __future__ import annotations

import math

import numpy as np

# ---------------------------------------------------------------------------
# Element formats  ([PF] commit "Gate split-KV off when kv_data_type is NVFP4":
# packed uint8 with a per-16-element FP8 block scale; [XQA] changelog:
# __nv_fp4_e2m1 elements, float4_e2m1fn_x2 containers)
# ---------------------------------------------------------------------------

E2M1_MAGNITUDE = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
E4M3_MAX = 448.0
BLOCK = 16  # head-dim elements per scale ([PF] "...split boundary never slices a scale block")


def e2m1_value(nibble):
    """Value of 4-bit e2m1 codes (any integer array; only the low 4 bits are used)."""
    nibble = np.asarray(nibble).astype(np.int64) & 0xF
    mag = E2M1_MAGNITUDE[nibble & 7]
    return np.where(nibble & 8, -mag, mag)


def e4m3_value(code):
    """Value of e4m3fn bytes as float64 (NaN for 0x7F and 0xFF)."""
    code = np.asarray(code).astype(np.int64) & 0xFF
    sign = np.where(code & 0x80, -1.0, 1.0)
    exp = (code >> 3) & 0xF
    man = code & 0x7
    normal = (1.0 + man / 8.0) * np.exp2(exp - 7.0)
    sub = (man / 8.0) * 2.0 ** -6
    val = np.where(exp == 0, sub, normal)
    val = np.where((exp == 15) & (man == 7), np.nan, val)
    return sign * val


# All non-negative finite e4m3 values, ordered, with their codes (code 0..126).
_E4M3_POS_CODES = np.arange(127, dtype=np.int64)
_E4M3_POS_VALUES = e4m3_value(_E4M3_POS_CODES)


def _round_to_grid(x, grid, codes):
    """Nearest grid value to each x >= 0, ties to the even code, saturating at the top.

    ``grid`` is increasing and ``codes`` are its codes; for both e2m1 and e4m3
    consecutive grid points have consecutive codes, so "even code" is the usual
    round-half-to-even on the significand.
    """
    x = np.asarray(x, dtype=np.float64)
    hi = np.searchsorted(grid, x, side="left")          # grid[hi-1] < x <= grid[hi]
    hi = np.clip(hi, 1, len(grid) - 1)
    lo = hi - 1
    d_lo = x - grid[lo]
    d_hi = grid[hi] - x
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (codes[hi] % 2 == 0))
    out = np.where(pick_hi, codes[hi], codes[lo])
    out = np.where(x >= grid[-1], codes[-1], out)       # satfinite
    out = np.where(x <= grid[0], codes[0], out)
    return out


def e4m3_round(x):
    """RNE to e4m3fn, saturating to 448, for x >= 0.  Returns codes (uint8)."""
    return _round_to_grid(x, _E4M3_POS_VALUES, _E4M3_POS_CODES).astype(np.uint8)


def e2m1_round(r):
    """RNE to the e2m1 magnitudes, saturating to 6, for r >= 0.  Returns codes 0..7."""
    return _round_to_grid(r, E2M1_MAGNITUDE, np.arange(8)).astype(np.uint8)


# ---------------------------------------------------------------------------
# Quantise / dequantise rows  ([XQA] changelog: tests' to_nvfp4 / nvfp4_to_float
# with a global scale; scale = amax / 6 with global scale 1 for the workloads)
# ---------------------------------------------------------------------------

def quantize(x, global_scale=1.0):
    """Quantise rows x[..., D] (D a multiple of 16) to NVFP4.

    Returns (packed uint8 [..., D/2], scale bytes uint8 [..., D/16]).
    Every block of 16 consecutive head-dim elements of one row gets its own scale.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    if d % BLOCK:
        raise ValueError("head dim must be a multiple of 16")
    g = float(global_scale)
    blocks = x.reshape(x.shape[:-1] + (d // BLOCK, BLOCK))
    amax = np.abs(blocks).max(axis=-1)
    sf = e4m3_round(amax / (6.0 * g))
    s = e4m3_value(sf)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(s > 0, np.abs(blocks) / (s * g), 0.0)
    mag = e2m1_round(r)
    sign = np.signbit(blocks).astype(np.uint8)
    nib = (sign << 3) | mag
    nib = nib.reshape(x.shape[:-1] + (d,))
    packed = (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)
    return packed, sf.astype(np.uint8)


def unpack_nibbles(packed):
    """uint8 [..., D/2] -> nibble codes [..., D] (low nibble first)."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed & 0xF
    out[..., 1::2] = packed >> 4
    return out


def dequantize(packed, sf, global_scale=1.0):
    """NVFP4 rows back to float64: e2m1(nibble) * e4m3(scale of its block) * g."""
    nib = unpack_nibbles(packed)
    vals = e2m1_value(nib)
    scale = np.repeat(e4m3_value(sf), BLOCK, axis=-1)
    return vals * scale * float(global_scale)


# ---------------------------------------------------------------------------
# FP8 e4m3 KV with a per-tensor scale  ([PF] commit "Gate split-KV off...": the
# FP8 and 16-bit KV types run the same prefill plan; dtype-aware skip commit: the
# float8_e4m3fn KV parametrisation)
# ---------------------------------------------------------------------------

def quantize_fp8(x, global_scale=1.0):
    """Rows x[..., D] to FP8 e4m3fn bytes: sign bit of x, magnitude RNE_e4m3(|x| / g)
    saturating at 448 (so -0 and tiny negatives give 0x80)."""
    x = np.asarray(x, dtype=np.float64)
    mag = e4m3_round(np.abs(x) / float(global_scale))
    sign = np.signbit(x).astype(np.uint8) << 7
    return (sign | mag).astype(np.uint8)


def dequantize_fp8(codes, global_scale=1.0):
    """FP8 e4m3fn bytes back to float64: e4m3(code) * g."""
    return e4m3_value(codes) * float(global_scale)


def dequantize_kv(data, sf, global_scale, kv_dtype):
    """Dequantised rows of either KV type (``sf`` is unused for FP8)."""
    if kv_dtype == "nvfp4":
        return dequantize(data, sf, global_scale)
    if kv_dtype == "fp8":
        return dequantize_fp8(data, global_scale)
    raise ValueError(kv_dtype)


# ---------------------------------------------------------------------------
# Paged cache reads  ([XQA] walkthrough: k_cache / v_cache with a page table and
# sequence lengths; [PF] independent K/V pools and strides)
# ---------------------------------------------------------------------------

def gather_pages(pool, page_table_row, kv_len, page_size, layout="HND"):
    """Rows of one request from a paged pool, in token order.

    pool: [pages, H, P, W] ("HND") or [pages, P, H, W] ("NHD").
    Token j lives at page page_table_row[j // P], slot j % P.
    Returns [kv_len, H, W].
    """
    j = np.arange(kv_len)
    pages = np.asarray(page_table_row)[j // page_size]
    slots = j % page_size
    if layout == "HND":
        return np.asarray(pool)[pages, :, slots, :]
    if layout == "NHD":
        return np.asarray(pool)[pages, slots, :, :]
    raise ValueError(layout)


# ---------------------------------------------------------------------------
# Attention  ([FIX] commit "...write lse...": lse is ln-sum-exp of the scaled
# scores, uniform scores give ln(seq_len); [PF] commit "Gate split-KV off...":
# decode and prefix-cache extend, qo_len << kv_len)
# ---------------------------------------------------------------------------

def attention(q, k, v, sm_scale, causal=False, mask=None):
    """Exact softmax attention of one request.

    q [n, Hq, Dk], k [L, Hkv, Dk], v [L, Hkv, Dv] (float64, already dequantised).
    Query row i sees keys j < L, and with ``causal`` only j <= i + (L - n); a boolean
    ``mask`` [n, L] (True = visible) replaces both rules.
    Returns O [n, Hq, Dv] and LSE [n, Hq] (natural log).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, hq, _ = q.shape
    L, hkv, _ = k.shape
    dv = v.shape[-1]
    group = hq // hkv
    o = np.zeros((n, hq, dv))
    lse = np.full((n, hq), -np.inf)
    if L == 0 or n == 0:
        return o, lse
    visible = np.ones((n, L), dtype=bool)
    if causal:
        visible = np.arange(L)[None, :] <= (np.arange(n)[:, None] + (L - n))
    if mask is not None:
        visible = np.asarray(mask, dtype=bool).reshape(n, L)
    for h in range(hq):
        g = h // group
        s = sm_scale * (q[:, h, :] @ k[:, g, :].T)          # [n, L]
        s = np.where(visible, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        has = np.isfinite(m[:, 0])
        m_safe = np.where(np.isfinite(m), m, 0.0)
        e = np.exp(s - m_safe)
        ell = e.sum(axis=1)
        with np.errstate(divide="ignore", invalid="ignore"):
            o_h = (e @ v[:, g, :]) / ell[:, None]
            lse_h = m_safe[:, 0] + np.log(ell)
        o[:, h, :] = np.where(has[:, None], o_h, 0.0)
        lse[:, h] = np.where(has, lse_h, -np.inf)
    return o, lse


def mask_segments(qo_lens, kv_lens):
    """Byte offset of each request's packed mask bits, and the total bytes."""
    sizes = [-(-int(q) * int(l) // 8) for q, l in zip(qo_lens, kv_lens)]
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    return off[:-1], int(off[-1])


def unpack_mask_segment(packed, byte_offset, q, L):
    """Request mask [q, L] from its packed bits: element e = i*L + j is bit e % 8 of
    byte byte_offset + e // 8."""
    e = np.arange(q * L, dtype=np.int64)
    byte = np.asarray(packed, dtype=np.uint8)[byte_offset + e // 8]
    return ((byte >> (e % 8).astype(np.uint8)) & 1).astype(bool).reshape(q, L)


def pack_masks(masks):
    """Boolean masks [q_b, L_b] of the requests -> packed bytes (each request's bits on
    their own, little-endian within a byte, padded to a byte)."""
    out = []
    for m in masks:
        bits = np.asarray(m, dtype=bool).ravel()
        nbytes = -(-bits.size // 8)
        buf = np.zeros(nbytes, dtype=np.uint8)
        for e in np.flatnonzero(bits):
            buf[e // 8] |= np.uint8(1 << (e % 8))
        out.append(buf)
    return np.concatenate(out) if out else np.zeros(0, dtype=np.uint8)


# ---------------------------------------------------------------------------
# Rotary position embedding  ([PF] commit "Address CodeRabbit review on
# flashinfer-ai#3684 (5 findings)", item init_rope_freq: the in-kernel rotary's
# frequency table has one entry per pair of QK head-dim elements, NUM_MMA_D_QK/2
# MMA tiles of them, and must span the QK dim also where the VO dim is smaller;
# pos_encoding_mode of the prefill paths)
# ---------------------------------------------------------------------------

def rope_frequencies(head_dim, theta=1e4, scale=1.0):
    """Angular frequency of each of the head_dim/2 element pairs:
    w_i = theta^(-2i / head_dim) / scale (radians per position)."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(float(theta), -2.0 * i / head_dim) / float(scale)


def apply_rope(x, positions, theta=1e4, scale=1.0):
    """Rotate rows x [n, H, D] (float64) at integer ``positions`` [n]: the pair
    (x_i, x_{i+D/2}) becomes (x_i cos a - x_{i+D/2} sin a, x_{i+D/2} cos a + x_i sin a)
    with a = pos * w_i, i < D/2."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    h = d // 2
    ang = np.asarray(positions, dtype=np.float64)[:, None] * rope_frequencies(d, theta, scale)[None, :]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def query_positions(q_len, kv_len):
    """Positions of a request's query rows: the last q_len of its kv_len positions."""
    return np.arange(q_len, dtype=np.int64) + (int(kv_len) - int(q_len))


def _rotate(q, k, kv_len, rope):
    """Q and K of one request rotated at their positions (rope = (theta, scale))."""
    if rope is None:
        return q, k
    theta, scale = rope
    return (apply_rope(q, query_positions(q.shape[0], kv_len), theta, scale),
            apply_rope(k, np.arange(k.shape[0]), theta, scale))


def paged_attention(q, k_pool, k_sf, v_pool, v_sf, page_table, kv_lens, qo_indptr,
                    page_size, sm_scale, causal=False, layout="HND",
                    k_global=1.0, v_global=1.0, rows=None, kv_dtype="nvfp4",
                    custom_mask=None, rope=None):
    """Batched attention over paged K/V (decode when every q_b is 1).

    q [sum q_b, Hq, Dk]; pools as in ``gather_pages`` with W = D/2 (NVFP4 data),
    D/16 (NVFP4 scales) or D (FP8 data; scales None).  ``rows`` optionally restricts
    the computation to a subset of requests (the other outputs stay NaN).
    ``custom_mask``: packed mask bytes of all requests (see ``mask_segments``), which
    then decide visibility in place of ``causal``.  ``rope`` = (theta, scale) rotates
    Q and the dequantised K at their positions first (``apply_rope``).  Returns
    O [sum q_b, Hq, Dv] and LSE [sum q_b, Hq].
    """
    q = np.asarray(q, dtype=np.float64)
    nq, hq, _ = q.shape
    dv = np.asarray(v_pool).shape[-1] * (2 if kv_dtype == "nvfp4" else 1)
    qo_lens = [int(qo_indptr[b + 1]) - int(qo_indptr[b]) for b in range(len(kv_lens))]
    seg = mask_segments(qo_lens, kv_lens)[0] if custom_mask is not None else None
    o = np.full((nq, hq, dv), np.nan)
    lse = np.full((nq, hq), np.nan)
    batch = len(kv_lens)

    def rows_of(pool, b, L):
        return None if pool is None else gather_pages(pool, page_table[b], L, page_size, layout)

    for b in (range(batch) if rows is None else rows):
        L = int(kv_lens[b])
        q0, q1 = int(qo_indptr[b]), int(qo_indptr[b + 1])
        k = dequantize_kv(rows_of(k_pool, b, L), rows_of(k_sf, b, L), k_global, kv_dtype)
        v = dequantize_kv(rows_of(v_pool, b, L), rows_of(v_sf, b, L), v_global, kv_dtype)
        m = None if seg is None else unpack_mask_segment(custom_mask, seg[b], q1 - q0, L)
        qb, k = _rotate(q[q0:q1], k, L, rope)
        o[q0:q1], lse[q0:q1] = attention(qb, k, v, sm_scale, causal, m)
    return o, lse


def ragged_attention(q, k_rows, k_sf, v_rows, v_sf, kv_indptr, qo_indptr, sm_scale,
                     causal=False, k_global=1.0, v_global=1.0, kv_dtype="nvfp4", rope=None):
    """Batched attention over ragged (non-paged) K/V: request b's keys are rows
    kv_indptr[b] .. kv_indptr[b+1]-1 of k_rows / v_rows [rows, Hkv, W] (and of the
    scale arrays for NVFP4); ``rope`` as in ``paged_attention``.  Returns
    O [sum q_b, Hq, Dv] and LSE [sum q_b, Hq]."""
    q = np.asarray(q, dtype=np.float64)
    nq, hq, _ = q.shape
    dv = np.asarray(v_rows).shape[-1] * (2 if kv_dtype == "nvfp4" else 1)
    o = np.full((nq, hq, dv), np.nan)
    lse = np.full((nq, hq), np.nan)
    for b in range(len(kv_indptr) - 1):
        a0, a1 = int(kv_indptr[b]), int(kv_indptr[b + 1])
        q0, q1 = int(qo_indptr[b]), int(qo_indptr[b + 1])
        k = dequantize_kv(np.asarray(k_rows)[a0:a1], None if k_sf is None else
                          np.asarray(k_sf)[a0:a1], k_global, kv_dtype)
        v = dequantize_kv(np.asarray(v_rows)[a0:a1], None if v_sf is None else
                          np.asarray(v_sf)[a0:a1], v_global, kv_dtype)
        qb, k = _rotate(q[q0:q1], k, a1 - a0, rope)
        o[q0:q1], lse[q0:q1] = attention(qb, k, v, sm_scale, causal)
    return o, lse


# ---------------------------------------------------------------------------
# Merge of partial states  ([XQA] changelog: mergeAndSaveOutTile combines the
# split-KV partial outputs)
# ---------------------------------------------------------------------------

def merge_states(o_parts, lse_parts):
    """Combine partial attention states computed over disjoint key sets.

    o_parts [n, ..., Dv], lse_parts [n, ...] -> (O [..., Dv], LSE [...]).
    lse = M + ln sum_c exp(lse_c - M) with M = max_c lse_c;
    O = sum_c exp(lse_c - lse) * O_c.  A part with lse = -inf contributes nothing;
    if every part is -inf the result is O = 0, LSE = -inf.
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    m = lse_parts.max(axis=0)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    w = np.where(np.isfinite(lse_parts), np.exp(lse_parts - m_safe), 0.0)
    total = w.sum(axis=0)
    with np.errstate(divide="ignore", invalid="ignore"):
        lse = np.where(finite, m_safe + np.log(total), -np.inf)
        o = np.where(finite[..., None], (w[..., None] * o_parts).sum(axis=0) / total[..., None], 0.0)
    return o, lse


# ---------------------------------------------------------------------------
# Split-KV chunking rules  ([PF] commit "Gate split-KV off...": the follow-up
# asks for 16-token-aligned chunk boundaries)
# ---------------------------------------------------------------------------

def check_chunks(kv_len, chunks, align=16):
    """Raise unless ``chunks`` [(begin, end), ...] tile [0, kv_len) in order with
    every inner boundary a multiple of ``align`` and no empty chunk (a request
    with kv_len 0 has exactly one empty chunk)."""
    chunks = [(int(a), int(b)) for a, b in chunks]
    if kv_len == 0:
        if chunks != [(0, 0)]:
            raise AssertionError(f"empty request must have one empty chunk, got {chunks}")
        return
    if not chunks or chunks[0][0] != 0 or chunks[-1][1] != kv_len:
        raise AssertionError(f"chunks {chunks} do not span [0, {kv_len})")
    for (a, b), (c, _) in zip(chunks, chunks[1:]):
        if b != c:
            raise AssertionError(f"gap or overlap at {b}/{c}")
    for a, b in chunks:
        if b <= a:
            raise AssertionError(f"empty chunk ({a}, {b})")
        if a % align:
            raise AssertionError(f"chunk start {a} not a multiple of {align}")
        if b != kv_len and b % align:
            raise AssertionError(f"chunk end {b} not a multiple of {align}")
