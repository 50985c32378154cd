"""CPU tests of the tuner's table handling and of the committed tile table (no GPU)."""
import json
import os

from block_scaled_w8a8_amd import sweep

HERE = os.path.dirname(os.path.abspath(__file__))
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
