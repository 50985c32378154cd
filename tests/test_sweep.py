"""CPU tests of the tuner's table handling and of the committed tile table (no GPU)."""
import json
import os

import pytest

from block_scaled_w8a8_amd import sweep

HERE = os.path.dirname(os.path.abspath(__file__))
REPO = os.path.dirname(HERE)
TABLE = os.path.join(os.path.dirname(HERE), "block_scaled_w8a8_amd", "tables", "gfx950.json")


def test_merge_keeps_untouched_batch_sizes():
    old = {"configs": {"1": {"bm": 16}, "64": {"bm": 64}, "4096": {"bm": 256}},
           "us": {"1": 27.0, "64": 35.0, "4096": 680.0}}
    new = {"configs": {"64": {"bm": 32}, "128": {"bm": 128}}, "us": {"64": 34.0, "128": 50.0}}
    sweep.merge_configs(old, new)
    assert list(new["configs"]) == ["1", "64", "128", "4096"]          # numeric order
    assert new["configs"]["64"] == {"bm": 32} and new["configs"]["1"] == {"bm": 16}
    assert new["us"] == {"1": 27.0, "64": 34.0, "128": 50.0, "4096": 680.0}


def test_committed_table_covers_the_grid(bfq):
    """Every committed entry has a config and a time for each bucket of the M (or token)
    grid, and the library accepts the whole table (it rejects tiles it has not compiled)."""
    table = json.load(open(TABLE))
    assert table["device"] == "gfx950" and table["entries"]
    grid = [str(m) for m in sweep.M_GRID]
    keys = set()
    for e in table["entries"]:
        assert list(e["configs"]) == grid, (e["N"], e["K"])
        assert list(e["us"]) == grid
        key = (e["N"], e["K"], e["dtype"], e.get("w_layout", "row_major"),
               e.get("scales", "fp32"), e.get("block_shape", [128, 128])[0], e.get("E", 0))
        assert key not in keys, key
        keys.add(key)
    assert bfq.bfq_load_tile_table(TABLE) >= 0
    bfq.bfq_load_tile_table(None)
    # a tuned dense shape and a tuned MoE shape are found (no default-rule warning)
    st, t = bfq.bfq_select_tile(4096, 24576, 7168, w_layout=bfq.BFQ_W_PACKED16)
    assert st == bfq.BFQ_OK and (t.bm, t.bn) == (256, 256)
    st, t = bfq.bfq_moe_select_tile(4096, 8, 256, 4096, 7168, w_layout=bfq.BFQ_W_PACKED16)
    assert st == bfq.BFQ_OK


def test_reference_key_matches_the_oracle_script():
    """The sweep reads the expected-value file under the same keys the oracle's
    sweep_reference script writes them."""
    from block_scaled_w8a8_amd import sweep
    from oracle import sweep_reference
    for args in ((24576, 7168, "fp8", "fp32", 64), (1536, 7168, "int8", "channel", 4096)):
        assert sweep.reference_key(*args) == sweep_reference.key(*args)


def test_meets_bar_is_the_parity_bar():
    """The sweep's gate: relative Frobenius <= 1e-3 and max |diff| <= 2^-7 * rms + 1e-3,
    both required; non-finite outputs fail."""
    import numpy as np
    from block_scaled_w8a8_amd import sweep
    ref = np.ones(100_000)
    bound = 1.0 / 128 + 1e-3
    assert sweep.meets_bar(ref.copy(), ref)
    one = ref.copy()
    one[3] += bound * (1 + 1e-6)
    assert not sweep.meets_bar(one, ref)
    one[3] = 1.0 - bound * (1 + 1e-6)
    assert not sweep.meets_bar(one, ref)
    assert not sweep.meets_bar(ref * (1 + 1.01e-3), ref)
    assert sweep.meets_bar(ref * (1 + 0.99e-3), ref)
    nan = ref.copy()
    nan[0] = np.nan
    assert not sweep.meets_bar(nan, ref)
    assert not sweep.meets_bar(ref[:10], ref)


def test_reference_file_round_trip(tmp_path, orc):
    """A small expected-value file: the sample positions lie in range, the values are the
    oracle's block GEMM at those positions, and the gate passes them and fails a perturbed
    copy."""
    import subprocess
    import sys
    import numpy as np
    from block_scaled_w8a8_amd import sweep, synth
    out = tmp_path / "ref.npz"
    subprocess.run([sys.executable, "-m", "oracle.sweep_reference", "--out", str(out), "--shapes",
                    "256,384", "--grid", "3", "40", "--samples", "100"], check=True, cwd=REPO)
    ref = sweep.Reference(str(out))
    x = synth.activations(40, 384, seed=0)
    qa, sa = orc.quant_groups(synth.bf16_bits(x))
    qw, sw = orc.quant_blocks(synth.weights(256, 384, seed=0).numpy())
    full, _ = orc.block_gemm(qa, sa, qw, sw)
    for M in (3, 40):
        ms, ns, vals = ref.get(256, 384, "fp8", "fp32", M)
        assert ms.size == 102 and (ms < M).all() and (ns < 256).all()
        full_m, _ = orc.block_gemm(qa[:M], sa[:M], qw, sw)
        assert np.array_equal(vals, full_m[ms, ns])
        assert np.array_equal(vals, full[ms, ns])          # rows nest across M
        assert sweep.meets_bar(vals, vals)
        bad = vals.copy()
        bad[0] += 1.0
        assert not sweep.meets_bar(bad, vals)
    with pytest.raises(SystemExit, match="oracle.sweep_reference"):
        ref.get(256, 384, "fp8", "fp32", 7)
