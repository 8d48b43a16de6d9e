"""bench.py's host logic (no GPU): the algorithmic byte and flop counts it
divides by the measured times, the single-GPU guard, and the rule that a
committed traffic record is used only for the workload and source it was
counted on."""
from __future__ import annotations

import os
import subprocess
import sys
from types import SimpleNamespace

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _batch(row_pos_per_req, c, k):
    rows = [t for req in row_pos_per_req for t in req]
    ptr = np.cumsum([0] + [len(req) for req in row_pos_per_req]).astype(np.int32)
    return SimpleNamespace(row_pos=np.array(rows, dtype=np.int32), req_row_ptr=ptr, num_req=len(row_pos_per_req),
                           num_rows=len(rows), c=c, k=k)


def test_headline_step_and_scorer_bytes():
    # 16 requests x 1 row at t = 81,919 (81,920 visible keys, c = 1), k = 2048:
    # keys 335,544,320 + q 16,384 + page table 81,920 + selection 131,072.
    inp = _batch([[81919]] * 16, c=1, k=2048)
    assert bench.step_bytes(inp) == 335_773_696
    # the scorer writes one FP32 score per visible block instead of the selection
    assert bench.scorer_bytes(inp) == 335_544_320 + 16_384 + 81_920 + 16 * 81920 * 4


def test_prefill_flops():
    # 8,192 rows at t = 57,344 .. 65,535, c = 4: 125,827,072 visible (row, block)
    # pairs, each 4 heads x 128 multiply-adds.
    inp = _batch([list(range(57344, 65536))], c=4, k=512)
    assert int(((inp.row_pos.astype(np.int64) + 1) // 4).sum()) == 125_827_072
    assert bench.prefill_flops(inp) == 128_846_921_728


def test_keys_counted_once_per_request():
    # Rows of one request share its keys: the longest row's range is read once.
    one = _batch([[4095], [8191]], c=4, k=512)
    shared = _batch([[4095, 8191]], c=4, k=512)
    per_key = 256
    assert bench.step_bytes(one) - bench.step_bytes(shared) == 1024 * per_key + (1024 // 16) * 4  # keys, page ids


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_traffic_record_only_for_its_workload_and_source():
    dig = bench.source_digest("score_decode.hip", "device.h")
    rec = bench.measured_traffic("score_decode", dig, "dsa_decode_16x80k")
    assert rec is None or rec > 0
    assert bench.measured_traffic("score_decode", dig, "qsa_decode_1x8k") is None
    assert bench.measured_traffic("score_decode", "0" * 16, "dsa_decode_16x80k") is None
