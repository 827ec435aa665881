"""The seeded input generators (no layer arithmetic lives there)."""
import numpy as np

import synth


def test_splitmix64_reference_outputs():
    # published splitmix64 reference sequence for seed 1234567
    ref = [6457827717110365317, 3203168211198807973, 9817491932198370423,
           4593380528125082431, 16408922859458223821]
    assert [int(v) for v in synth.hash_words(1234567, 0, 5)] == ref


def test_byte_streams_are_position_addressed():
    k = synth.stream_key(3, 1, synth.DOWN_PACKED)
    full = synth.packed_bytes(k, 0, 1000)
    for s, n in ((0, 8), (5, 17), (13, 300), (992, 8)):
        assert np.array_equal(synth.packed_bytes(k, s, n), full[s:s + n])
    sc = synth.scale_bytes(k, 0, 5000)
    assert sc.min() == 120 and sc.max() == 126
    assert np.array_equal(synth.scale_bytes(k, 1234, 50), sc[1234:1284])
    # both nibbles take all 16 codes
    assert len(set((full & 15).tolist())) == 16 and len(set((full >> 4).tolist())) == 16


def test_bf16_rounding():
    v = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 3.0e38, 1e-40], np.float32)
    b = synth.bf16_bits(v)
    assert list(b[:4]) == [0x3F80, 0x3F80, 0x3F82, 0xC020]
    back = synth.bf16_to_f32(b)
    assert back[0] == 1.0 and back[3] == -2.5


def test_expert_host_layout():
    spec = synth.tiny_spec(seed=9)
    h = synth.expert_host(spec, [2, 5])
    assert h["gate_packed"].shape == (2, spec.inter, spec.hidden // 2)
    assert h["down_scales"].shape == (2, spec.hidden, spec.inter // 32)
    k = synth.stream_key(9, 0, synth.UP_PACKED)
    n = spec.inter * spec.hidden // 2
    assert np.array_equal(h["up_packed"][1].ravel(), synth.packed_bytes(k, 5 * n, n))


def test_zipf_prior_column():
    spec = synth.LayerSpec(hidden=64, inter=64, n_experts=16, topk=2, routing="zipf", seed=1)
    x = synth.make_x(spec, 3)
    Wr = synth.make_router(spec)
    assert np.all(synth.bf16_to_f32(x[:, 0]) == 1.0)
    col = synth.bf16_to_f32(Wr[:, 0])
    assert col.max() == 0.0 and np.sum(col == 0.0) == 1
