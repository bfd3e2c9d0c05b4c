"""CPU replica of how the attention kernel walks the cached keys of a frame range
(nomas_segment_attention_frames), checked for exact coverage and in-bounds reads.

The range [first, first + n) of retained frames becomes physical cache tokens:
all retained frames in slot order when n is every retained frame, otherwise the
run [s*tpf, (s + na)*tpf) from slot s = first mod capacity and, when the range
wraps round the ring, the run [0, nb*tpf). Tiles of BC keys: the full tiles of
the first run, those of the second, then each run's partial tail; a tail whose
BC rows would pass token_pitch (round_up(capacity*tpf, 128)) is moved back to
end there, its valid rows starting at an offset. The claim: every tile reads
rows inside [0, token_pitch) and the valid rows of all tiles are exactly the
range's tokens, each once. (The replica restates the kernel's index arithmetic;
the GPU tests check the kernel's results against the oracle.)"""

import pytest


def _pitch(tpf, cap):
    return (cap * tpf + 127) // 128 * 128


def _runs(fw, cap, tpf, first, n):
    valid = min(fw, cap)
    if n == valid:
        return 0, valid * tpf, 0
    s = first % cap
    na = min(n, cap - s)
    return s * tpf, na * tpf, (n - na) * tpf


def _tiles(a0, na, nb, bc, pitch):
    full_a = na // bc
    full_c = full_a + nb // bc
    n_tiles = full_c + (na % bc != 0) + (nb % bc != 0)
    out = []
    for t in range(n_tiles):
        lo = 0
        if t < full_a:
            k0, n = a0 + t * bc, bc
        elif t < full_c:
            k0, n = (t - full_a) * bc, bc
        elif t == full_c and na % bc:
            k0, n = a0 + full_a * bc, na % bc
        else:
            k0, n = nb // bc * bc, nb % bc
        if k0 + bc > pitch:
            lo, k0 = k0 - (pitch - bc), pitch - bc
        out.append((k0, n, lo))
    return out


@pytest.mark.parametrize("tpf", [1, 5, 24, 40, 100, 960])
@pytest.mark.parametrize("cap", [1, 3, 5, 26])
@pytest.mark.parametrize("bc", [64, 128])
def test_tiles_cover_the_range_exactly_inside_the_head(tpf, cap, bc):
    if cap * tpf > 5000:
        pytest.skip("covered by the smaller rings (seconds, not minutes, of CPU)")
    pitch = _pitch(tpf, cap)
    for fw in range(0, 2 * cap + 3):
        valid = min(fw, cap)
        for first in range(fw - valid, fw + 1):
            for n in range(0, fw - first + 1):
                a0, na, nb = _runs(fw, cap, tpf, first, n)
                if n == valid:
                    want = list(range(valid * tpf))
                else:
                    want = sorted((f % cap) * tpf + i for f in range(first, first + n) for i in range(tpf))
                got = []
                for k0, nv, lo in _tiles(a0, na, nb, bc, pitch):
                    assert 0 <= k0 and k0 + bc <= pitch, (fw, first, n, k0)
                    assert 0 <= lo and lo + nv <= bc
                    got += range(k0 + lo, k0 + lo + nv)
                assert sorted(got) == want, (fw, first, n)
