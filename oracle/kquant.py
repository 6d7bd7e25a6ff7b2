"""GGUF Q4_K / Q5_K / Q6_K super-block formats, decoded exactly to float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources.
  * OpenVINO PR #39119 "FullyConnectedGGUF", sections "Why a new primitive"
    (weights are byte rows of K/256*block_bytes) and "Transformation" (Q6_K
    regroup into the planes QL[nblk][128] | QH[nblk][64] | SC[nblk][16] |
    D[nblk], unchanged in size and contents).
  * onnxruntime-mobius "GGUF Support Proposal", section 1.2 (Q5_K is the
    5-bit and Q6_K the 6-bit K-quant, 256 values per super-block) and
    section 7.3 (the K-quant header d | dmin | 12 packed 6-bit scale/min
    bytes, and the roles sub_scale = sc*d, sub_min = m*dmin, value =
    q*sub_scale - sub_min).
  * onnxruntime-mobius "GGUF Support Proposal", section 7.3 (Q4_K): the
    144-byte struct d | dmin | scales[12] | qs[128], 32-value sub-blocks with
    a 6-bit scale and a 6-bit min each, value = q*sc*d - m*dmin.
  Q5_K weights are w = d*sc_j*q - dmin*m_j with q in [0,31]; Q4_K weights
  have the same form with q in [0,15]; Q6_K weights are w = d*sc_s*(q - 32)
  with q in [0,63] and a signed 8-bit scale per 16 values.

Readings where the pages are silent (bit positions are not printed; these
follow the GGUF on-disk convention of the reference runtime the pages name):
  Q5_K  bytes 0-1 d, 2-3 dmin, 4-15 scales, 16-47 qh, 48-175 qs.
        Sub-block j = i//32 of value i.  Low nibble: qs[32*(i//64) + i%32],
        low half if (i%64) < 32 else high half.  Fifth bit: bit j of
        qh[i%32].  6-bit fields, b = the 12 scale bytes:
          j < 4 : sc_j = b[j] & 63,  m_j = b[j+4] & 63
          j >= 4: sc_j = (b[j+4] & 15) | (b[j-4] >> 6) << 4
                  m_j  = (b[j+4] >> 4) | (b[j]   >> 6) << 4
  Q4_K  bytes 0-1 d, 2-3 dmin, 4-15 scales (packed as for Q5_K), 16-143 qs.
        Code of value i: qs[16 + 32*(i//64) + i%32] (block byte offset), low
        half if (i%64) < 32 else high half; sub-block j = i//32.
  Q6_K  bytes 0-127 ql, 128-191 qh, 192-207 sc (int8), 208-209 d.
        Value i: h = i//128, r = i%128, g = r//32, l = r%32.
        Low nibble: ql[64h + 32*(g%2) + l] >> 4*(g//2) & 15.
        High pair: qh[32h + l] >> 2g & 3.  Scale index s = i//16.
  Q6_K therefore has 16 sub-blocks of 16 values (16 scale bytes), not the
  "8 sub-blocks of 32" the proposal's section 1.2 states for all K-quants.
"""

from __future__ import annotations

import numpy as np

QK = 256
Q4K_BYTES = 144
Q5K_BYTES = 176
Q6K_BYTES = 210


def _f16_at(blk: np.ndarray, off: int) -> np.ndarray:
    """f16 little-endian at byte offset `off` of each block, as float64."""
    two = np.ascontiguousarray(blk[..., off:off + 2])
    return two.view(np.float16)[..., 0].astype(np.float64)


# ----------------------------------------------------------------- Q5_K ----

def q5k_scale_min(blk: np.ndarray):
    """(sc[..., 8], m[..., 8]) int64: the eight 6-bit scales and mins."""
    b = blk[..., 4:16].astype(np.int64)
    sc = np.empty(blk.shape[:-1] + (8,), dtype=np.int64)
    m = np.empty_like(sc)
    for j in range(8):
        if j < 4:
            sc[..., j] = b[..., j] & 63
            m[..., j] = b[..., j + 4] & 63
        else:
            sc[..., j] = (b[..., j + 4] & 15) | ((b[..., j - 4] >> 6) << 4)
            m[..., j] = (b[..., j + 4] >> 4) | ((b[..., j] >> 6) << 4)
    return sc, m


def q5k_codes(blk: np.ndarray) -> np.ndarray:
    """int64[..., 256]: the 5-bit code q_i in [0, 31] of every value."""
    qh = blk[..., 16:48].astype(np.int64)
    qs = blk[..., 48:176].astype(np.int64)
    q = np.empty(blk.shape[:-1] + (QK,), dtype=np.int64)
    for i in range(QK):
        j, l = i // 32, i % 32
        byte = qs[..., 32 * (i // 64) + l]
        low = (byte & 15) if (i % 64) < 32 else (byte >> 4)
        high = (qh[..., l] >> j) & 1
        q[..., i] = low + 16 * high
    return q


def decode_q5k(blk: np.ndarray) -> np.ndarray:
    """float64[..., 256]: w_i = d*sc_j*q_i - dmin*m_j, j = i//32 (exact)."""
    assert blk.shape[-1] == Q5K_BYTES
    d = _f16_at(blk, 0)[..., None]
    dmin = _f16_at(blk, 2)[..., None]
    sc, m = q5k_scale_min(blk)
    q = q5k_codes(blk).astype(np.float64)
    j = np.arange(QK) // 32
    return d * sc[..., j].astype(np.float64) * q - dmin * m[..., j].astype(np.float64)


# ----------------------------------------------------------------- Q4_K ----

def q4k_scale_min(blk: np.ndarray):
    """(sc[..., 8], m[..., 8]) int64 of a Q4_K block: the header (d, dmin,
    12 scale bytes) is laid out exactly as Q5_K's, so the fields are too."""
    return q5k_scale_min(blk)


def q4k_codes(blk: np.ndarray) -> np.ndarray:
    """int64[..., 256]: the 4-bit code q_i in [0, 15] of every value."""
    qs = blk[..., 16:144].astype(np.int64)
    q = np.empty(blk.shape[:-1] + (QK,), dtype=np.int64)
    for i in range(QK):
        byte = qs[..., 32 * (i // 64) + i % 32]
        q[..., i] = (byte & 15) if (i % 64) < 32 else (byte >> 4)
    return q


def decode_q4k(blk: np.ndarray) -> np.ndarray:
    """float64[..., 256]: w_i = q_i*(sc_j*d) - m_j*dmin, j = i//32 (exact)."""
    assert blk.shape[-1] == Q4K_BYTES
    d = _f16_at(blk, 0)[..., None]
    dmin = _f16_at(blk, 2)[..., None]
    sc, m = q4k_scale_min(blk)
    q = q4k_codes(blk).astype(np.float64)
    j = np.arange(QK) // 32
    return q * (sc[..., j].astype(np.float64) * d) - m[..., j].astype(np.float64) * dmin


# ----------------------------------------------------------------- Q6_K ----

def q6k_codes(blk: np.ndarray) -> np.ndarray:
    """int64[..., 256]: the 6-bit code q_i in [0, 63] of every value."""
    ql = blk[..., 0:128].astype(np.int64)
    qh = blk[..., 128:192].astype(np.int64)
    q = np.empty(blk.shape[:-1] + (QK,), dtype=np.int64)
    for i in range(QK):
        h, r = i // 128, i % 128
        g, l = r // 32, r % 32
        low = (ql[..., 64 * h + 32 * (g % 2) + l] >> (4 * (g // 2))) & 15
        high = (qh[..., 32 * h + l] >> (2 * g)) & 3
        q[..., i] = low + 16 * high
    return q


def q6k_scales(blk: np.ndarray) -> np.ndarray:
    """int64[..., 16]: the signed 8-bit sub-block scales."""
    return np.ascontiguousarray(blk[..., 192:208]).view(np.int8).astype(np.int64)


def decode_q6k(blk: np.ndarray) -> np.ndarray:
    """float64[..., 256]: w_i = d*sc_{i//16}*(q_i - 32) (exact)."""
    assert blk.shape[-1] == Q6K_BYTES
    d = _f16_at(blk, 208)[..., None]
    sc = q6k_scales(blk)
    q = q6k_codes(blk)
    s = np.arange(QK) // 16
    return d * sc[..., s].astype(np.float64) * (q - 32).astype(np.float64)


# ------------------------------------------------------------ matrices ----

def block_bytes(qtype: str) -> int:
    return {"q4_k": Q4K_BYTES, "q5_k": Q5K_BYTES, "q6_k": Q6K_BYTES}[qtype]


def as_blocks(w_bytes: np.ndarray, qtype: str) -> np.ndarray:
    """u8[N, K/256*B] -> u8[N, K/256, B]."""
    B = block_bytes(qtype)
    N = w_bytes.shape[0]
    assert w_bytes.shape[1] % B == 0
    return w_bytes.reshape(N, w_bytes.shape[1] // B, B)


def dequantize(w_bytes: np.ndarray, qtype: str) -> np.ndarray:
    """u8[N, K/256*B] -> float64[N, K], exact."""
    blk = as_blocks(w_bytes, qtype)
    dec = {"q4_k": decode_q4k, "q5_k": decode_q5k, "q6_k": decode_q6k}[qtype]
    N, nb = blk.shape[:2]
    return dec(blk).reshape(N, nb * QK)


# ---------------------------------------------------- Q6_K plane regroup ----

def q6k_regroup(w_bytes: np.ndarray) -> np.ndarray:
    """u8[N, K/256*210] -> u8[210*nblk]: QL | QH | SC | D planes.

    Blocks are taken in row-major (n, kb) order; each plane is the
    concatenation of that field over all nblk blocks, with no padding, so the
    byte count is unchanged (OpenVINO PR #39119, section Transformation).
    """
    blk = w_bytes.reshape(-1, Q6K_BYTES)
    return np.concatenate([
        blk[:, 0:128].reshape(-1),
        blk[:, 128:192].reshape(-1),
        blk[:, 192:208].reshape(-1),
        blk[:, 208:210].reshape(-1),
    ])


def q6k_ungroup(planes: np.ndarray, N: int, K: int) -> np.ndarray:
    """Inverse of q6k_regroup: planes -> u8[N, K/256*210]."""
    nblk = N * (K // QK)
    assert planes.size == nblk * Q6K_BYTES
    o = 0
    out = np.empty((nblk, Q6K_BYTES), dtype=np.uint8)
    for lo, hi in ((0, 128), (128, 192), (192, 208), (208, 210)):
        w = hi - lo
        out[:, lo:hi] = planes[o:o + w * nblk].reshape(nblk, w)
        o += w * nblk
    return out.reshape(N, (K // QK) * Q6K_BYTES)


# --------------------------------------------- encoders (hand-built blocks) --

def _pack_scale_min(sc, m) -> list:
    """The 12 scale bytes of a Q4_K / Q5_K header from 8 scales and 8 mins
    (6 bits each): low 6 bits of sc_0..3 and m_0..3 in bytes 0-3 and 4-7,
    the low nibbles of sc_4..7 | m_4..7 << 4 in bytes 8-11, and the top two
    bits of sc_4..7 / m_4..7 in bits 6-7 of bytes 0-3 / 4-7."""
    b = [0] * 12
    for j in range(4):
        b[j] |= sc[j] & 63
        b[j + 4] |= m[j] & 63
    for j in range(4, 8):
        b[j + 4] |= (sc[j] & 15) | ((m[j] & 15) << 4)
        b[j - 4] |= (sc[j] >> 4) << 6
        b[j] |= (m[j] >> 4) << 6
    return b


def encode_q5k(d: float, dmin: float, sc, m, q) -> np.ndarray:
    """Build one Q5_K block from fields: d, dmin (f16), sc/m (8 x 6-bit),
    q (256 x 5-bit codes).  Inverse of the decoder's field extraction."""
    sc = [int(x) for x in sc]
    m = [int(x) for x in m]
    q = [int(x) for x in q]
    assert len(sc) == 8 and len(m) == 8 and len(q) == QK
    assert all(0 <= x < 64 for x in sc + m) and all(0 <= x < 32 for x in q)
    out = np.zeros(Q5K_BYTES, dtype=np.uint8)
    out[0:2] = np.array([d], dtype=np.float16).view(np.uint8)
    out[2:4] = np.array([dmin], dtype=np.float16).view(np.uint8)
    out[4:16] = _pack_scale_min(sc, m)
    for i in range(QK):
        j, l = i // 32, i % 32
        low, high = q[i] & 15, q[i] >> 4
        k = 48 + 32 * (i // 64) + l
        out[k] |= low if (i % 64) < 32 else (low << 4)
        out[16 + l] |= high << j
    return out


def encode_q4k(d: float, dmin: float, sc, m, q) -> np.ndarray:
    """Build one Q4_K block from d, dmin (f16), sc/m (8 x 6-bit) and q
    (256 x 4-bit codes), field by field."""
    sc = [int(x) for x in sc]
    m = [int(x) for x in m]
    q = [int(x) for x in q]
    assert len(sc) == 8 and len(m) == 8 and len(q) == QK
    assert all(0 <= x < 64 for x in sc + m) and all(0 <= x < 16 for x in q)
    out = np.zeros(Q4K_BYTES, dtype=np.uint8)
    out[0:2] = np.array([d], dtype=np.float16).view(np.uint8)
    out[2:4] = np.array([dmin], dtype=np.float16).view(np.uint8)
    out[4:16] = _pack_scale_min(sc, m)
    for c in range(4):                 # 64-value chunk c: qs[32c + l]
        for l in range(32):
            out[16 + 32 * c + l] = q[64 * c + l] | (q[64 * c + 32 + l] << 4)
    return out


def encode_q6k(d: float, sc, q) -> np.ndarray:
    """Build one Q6_K block from d (f16), sc (16 x int8), q (256 x 6-bit)."""
    sc = [int(x) for x in sc]
    q = [int(x) for x in q]
    assert len(sc) == 16 and len(q) == QK
    assert all(-128 <= x < 128 for x in sc) and all(0 <= x < 64 for x in q)
    out = np.zeros(Q6K_BYTES, dtype=np.uint8)
    for i in range(QK):
        h, r = i // 128, i % 128
        g, l = r // 32, r % 32
        out[64 * h + 32 * (g % 2) + l] |= (q[i] & 15) << (4 * (g // 2))
        out[128 + 32 * h + l] |= (q[i] >> 4) << (2 * g)
    out[192:208] = np.array(sc, dtype=np.int8).view(np.uint8)
    out[208:210] = np.array([d], dtype=np.float16).view(np.uint8)
    return out
