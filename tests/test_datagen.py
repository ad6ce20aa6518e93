"""Host-side input tooling: generators, index builder, index file round trip."""
import numpy as np

from approximate_nearest_neighbour_amd import datagen as G
from oracle import oracle as O


def test_zipf_sizes_shape():
    s = G.zipf_sizes(1_000_000_000, 262_144)
    assert s.sum() == 1_000_000_000
    assert np.all(np.diff(s) <= 0)
    assert s[0] == 129_656_229 and s[-1] == 142
    assert int(np.median(s)) == 304


def test_tiny_build_and_file_round_trip(tmp_path):
    w = G.tiny()
    idx = w.index
    assert idx.codes.shape == (10_000, 4) and idx.list_sizes.sum() == 10_000
    assert sorted(idx.ids.tolist()) == list(range(10_000))
    p = str(tmp_path / "tiny.ivfpq")
    G.write_index(p, idx)
    back = G.read_index(p)
    other = O.read_index_file(p)           # the oracle's own reader
    for name in ("centroids", "codebooks", "list_sizes", "codes", "ids"):
        assert np.array_equal(getattr(back, name), getattr(idx, name))
        assert np.array_equal(other[name], getattr(idx, name))


def test_generators_are_seeded():
    a = G.tiny()
    b = G.tiny()
    assert np.array_equal(a.queries, b.queries)
    assert np.array_equal(a.index.codes, b.index.codes)


def test_bf16_rounding_of_inputs():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.005859375], dtype=np.float32)
    back = G.bf16_bits_to_f32(G.to_bf16_bits(x))
    ref = np.array([1.0, 1.0, 1.015625, -2.5, 1.0078125], dtype=np.float32)
    assert np.array_equal(back, ref)
