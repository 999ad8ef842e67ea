"""The gated-logit and block-sparse oracles against cases worked by hand from the
definitions (tests/golden/gated_toy.json, block_toy.json)."""
import numpy as np

from oracle import blocksparse, sas
from oracle.numerics import bf16_to_f32
from tests import golden_variants as gv


def test_gated_toy_by_hand():
    g = gv.load("gated_toy")
    q, K, V = gv.padded_bits(g["q_heads"]), gv.padded_bits(g["K"]), gv.padded_bits(g["V"])
    u = np.array([gv.value(x) for x in g["u"]], dtype=np.float32)
    for c in g["cases"]:
        out, idx, _ = sas.gated_decode_unit(q, K, V, u, g["n"], g["unit_size"], g["k_units"], c["lambda"], 1.0)
        assert list(idx) == g["idx"]
        assert np.max(np.abs(out[:, :4] - gv.matrix(c["out"]))) < 1e-6
        assert np.all(out[:, 4:] == 0)


def test_block_toy_by_hand():
    g = gv.load("block_toy")
    q, K, V = gv.padded_bits(g["q_heads"]), gv.padded_bits(g["K"]), gv.padded_bits(g["V"])
    bs, n = g["block_size"], g["n"]
    kc = blocksparse.block_keys(K, n, bs)
    kcv = bf16_to_f32(kc)
    out, idx, blocks, s = blocksparse.decode_unit(q, K, V, kcv, n, bs, g["k_blocks"], g["n_init"], g["n_local"],
                                                  1.0)
    assert np.allclose(s[1:], [gv.value(x) for x in g["scores"]], rtol=1e-12)
    assert list(idx) == g["idx"]
    assert np.max(np.abs(out[:, :4] - gv.matrix(g["out"]))) < 1e-12
    # the INT4 selector cache keeps the same order here
    codes, scales = blocksparse.int4_quantize(kc)
    out4, idx4, _, _ = blocksparse.decode_unit(q, K, V, blocksparse.int4_dequantize(codes, scales), n, bs,
                                               g["k_blocks"], g["n_init"], g["n_local"], 1.0)
    assert list(idx4) == g["idx"]
