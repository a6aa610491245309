"""Host checks of two integer quotients the kernels take in fp32 instead of
by integer division (no GPU): trunc((v + 1/2) * rcp(d)) equals v // d over
the whole range each kernel uses it on, with the reciprocal rounded to fp32
as the kernels round it.  A miss here would put a cos/sin value, or a row,
under the wrong token."""

import numpy as np


def _quotients_exact(vmax, dmax):
    v = np.arange(vmax, dtype=np.int64)
    vf = v.astype(np.float32) + np.float32(0.5)
    for d in range(1, dmax + 1):
        inv = np.float32(1.0) / np.float32(d)
        q = np.trunc(vf * inv).astype(np.int64)
        bad = np.nonzero(q != v // d)[0]
        if bad.size:
            return d, int(v[bad[0]])
    return None


def test_cos_sin_value_codes():
    # token of value v = lane + 64 k (k < 4) among h <= 128 frequencies per token
    assert _quotients_exact(256, 128) is None


def test_row_to_token():
    # token of row rr < 2 * 2048 + 64 in a block of tokens of R <= 2048 rows
    assert _quotients_exact(2 * 2048 + 64, 2048) is None


def test_the_check_can_fail():
    # the same quotient without the half offset misses (v = d * n lands on a
    # rounding of n - epsilon for some d), so the checks above are not vacuous
    v = np.arange(4160, dtype=np.int64)
    misses = 0
    for d in range(1, 2049):
        inv = np.float32(1.0) / np.float32(d)
        q = np.trunc(v.astype(np.float32) * inv).astype(np.int64)
        misses += int(np.count_nonzero(q != v // d))
    assert misses > 0


def _lane_chunk(i, C, E, rotary_dim, interleaved):
    """Chunk held by lane position i of a row (the kernels' lane layout):
    half-split pairs put the two halves of every rotated pair in mirrored
    lanes, unrotated chunks in between; interleaved pairs keep chunk i."""
    if interleaved:
        return i
    hc = (rotary_dim // 2) // E
    if i < hc:
        return i
    if i >= C - hc:
        return C - 1 - i + hc
    return hc + i


def _lane_of_chunk(jc, C, E, rotary_dim, interleaved):
    """The closed form the norm-group backward uses to find the lane position
    holding chunk jc when it sums the weight-gradient slots."""
    if interleaved:
        return jc
    hc = (rotary_dim // 2) // E
    if jc < hc:
        return jc
    if jc < 2 * hc:
        return C - 1 + hc - jc
    return jc - hc


def test_lane_of_chunk_inverts_the_lane_layout():
    # every head size, element width (bf16: 8 per chunk, fp32: 4) and rotary
    # width the kernels accept (multiples of 16 up to head_dim)
    for D in (64, 128, 256):
        for E in (8, 4):
            C = D // E
            for R in range(0, D + 1, 16):
                for il in (False, True):
                    chunks = [_lane_chunk(i, C, E, R, il) for i in range(C)]
                    assert sorted(chunks) == list(range(C)), (D, E, R, il)
                    for i, jc in enumerate(chunks):
                        assert _lane_of_chunk(jc, C, E, R, il) == i, (D, E, R, il, jc)
