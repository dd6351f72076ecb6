"""Host-side layouts (include/leapquant.h: lq_state.codes, and the buffered
key rows of lq_state.ent_k): the test helpers that pack and unpack device
bytes, checked against the layout definitions written out by hand (CPU only)."""
import numpy as np
import pytest

from tests import gpu_helpers as gh

QMAX = {8: 127, 6: 31, 4: 7}


@pytest.mark.parametrize("bits", [8, 6, 4])
@pytest.mark.parametrize("d", [32, 64, 128])
def test_pack_unpack_round_trip(bits, d):
    rng = np.random.default_rng(bits * 1000 + d)
    Q = QMAX[bits]
    C = rng.integers(-Q, Q + 1, size=(3, d, d)).astype(np.int32)
    C[0, 0, :] = Q
    C[0, 1, :] = -Q
    raw = gh.pack_codes(C, bits)
    assert raw.shape == (3, d, d * bits // 8)
    assert np.array_equal(gh.unpack_codes(raw, bits, d), C)


def _code_by_definition(head: bytes, j: int, i: int, bits: int, d: int) -> int:
    """Code of value column j, key channel i from one head's bytes, read off
    the header's layout definition one field at a time."""
    if bits == 8:
        b = head[j * d + i]
        return b - 256 if b >= 128 else b
    nib = (head[j * (d // 2) + i // 2] >> (4 * (i % 2))) & 0xF
    hi = nib - 16 if nib >= 8 else nib
    if bits == 4:
        return hi
    nj = d // 16
    w = d * d // 2 + 4 * (((j % 16) * nj + i // 16) * nj + j // 16)
    word = int.from_bytes(head[w: w + 4], "little")
    c = i % 16
    p = c // 2 if c % 2 == 0 else 8 + c // 2
    lo = (word >> (8 * (p % 4) + 2 * (p // 4))) & 3
    return 4 * hi + lo


@pytest.mark.parametrize("bits", [8, 6, 4])
@pytest.mark.parametrize("d", [32, 64])
def test_layout_matches_definition(bits, d):
    rng = np.random.default_rng(7)
    Q = QMAX[bits]
    C = rng.integers(-Q, Q + 1, size=(1, d, d)).astype(np.int32)   # math layout [d_k][d_v]
    head = bytes(gh.pack_codes(C, bits).view(np.uint8).reshape(-1))
    for j in range(d):
        for i in range(d):
            assert _code_by_definition(head, j, i, bits, d) == C[0, i, j], (bits, i, j)


def test_six_bit_split():
    """code = 4 hi + lo with hi = floor(code / 4) in [-8, 7] and lo in [0, 3]."""
    for code in range(-31, 32):
        hi, lo = code >> 2, code & 3
        assert -8 <= hi <= 7 and 0 <= lo <= 3 and 4 * hi + lo == code


# ---- buffered key rows (include/leapquant.h, lq_state.ent_k): with bf16
# activations a buffered token's row holds its bf16 key in its first d * 2
# bytes; fp32 rows otherwise


def _dims(d, bf16, r=2, w=5):
    from linear_attention_recurrent_kda_amd import leapquant as lqk
    return lqk.Dims(batch=1, heads=3, d=d, w_max=w, n_comp=r, bf16=bf16)


@pytest.mark.parametrize("d", [32, 64, 128])
def test_bf16_key_rows_by_definition(d):
    dims = _dims(d, True)
    rng = np.random.default_rng(d)
    bits = rng.integers(0, 1 << 16, size=(3, dims.w_max, d), dtype=np.uint32)
    bits[(bits & 0x7F80) == 0x7F80] = 0x3F80  # no NaN/Inf patterns
    k = (bits << 16).view(np.float32)          # bf16 values as fp32
    rows = gh.buf_key_rows(k, dims)
    assert rows.shape == k.shape and rows.dtype == np.float32
    raw = rows.view(np.uint8).reshape(3, dims.w_max, 4 * d)
    for h in range(3):
        for e in range(dims.w_max):
            for c in (0, 1, d // 2, d - 1):
                b = int(bits[h, e, c])
                # channel c at bytes 2c, 2c + 1 of the row, little-endian
                assert raw[h, e, 2 * c] == b & 0xFF and raw[h, e, 2 * c + 1] == b >> 8
            assert not raw[h, e, 2 * d:].any()     # the row's second half is unused
    ent = np.zeros((3, dims.n_comp + dims.w_max, d), np.float32)
    ent[:, :dims.n_comp] = 0.25                  # compensator rows stay fp32
    ent[:, dims.n_comp:] = rows
    back = gh.buf_keys_f32(ent, dims)
    assert np.array_equal(back.view(np.uint32), k.view(np.uint32))


def test_key_rows_fp32_and_bf16_values_only():
    k = np.linspace(-1, 1, 3 * 5 * 32, dtype=np.float32).reshape(3, 5, 32)
    assert np.array_equal(gh.buf_key_rows(k, _dims(32, False)), k)  # fp32 activations: rows as they are
    with pytest.raises(AssertionError):
        gh.buf_key_rows(k + np.float32(1e-3), _dims(32, True))      # not bf16 values
