"""The benchmark's byte/FLOP accountant reproduces the page's own table.

"[Kimi-K3 MLA TP8] MLA performance", Sec. 5.3 "Strongly memory-bound": slot
counts -> KV MiB, index MiB, GFLOP (16 padded / 12 useful heads), FLOP/byte,
GB per 24-layer step and the 8 TB/s floor.  Tolerances are the page's rounding.
"""

import pytest

import workloads
from workloads import accounting as acc

MIB = 1 << 20


@pytest.mark.parametrize("case", ["c16", "c24"])
def test_accountant_reproduces_issue_table(golden, case):
    g = golden("issue_traffic.json")
    c = g["cases"][case]
    n, B = c["slots"], c["batch"]
    # lengths only matter through their sum (qlen 1)
    lengths = [n // B] * (B - 1) + [n - (n // B) * (B - 1)]
    qlens = [1] * B
    kv = n * acc.row_bytes("fp8")
    assert abs(kv / MIB - c["kv_mib"]) < 0.5
    assert abs(n * acc.INDEX_BYTES / MIB - c["index_mib"]) < 0.05
    assert B * 16 * 576 / 1024 == c["q_kib"] and B * 16 * 512 * 2 / 1024 == c["o_kib"]
    fl = acc.decode_flops(lengths, qlens, 16)
    assert abs(fl / 1e9 - c["gflop_padded"]) < 0.05
    assert abs(acc.decode_flops(lengths, qlens, 12) / 1e9 - c["gflop_useful"]) < 0.05
    by = acc.decode_bytes(lengths, qlens, 16, "fp8")
    assert abs(fl / by - c["flop_per_byte"]) < 1.0
    # The page's per-step total sums the gathered rows and their indices; the
    # accountant also counts q in / o out (0.06% more), shown separately.
    gathered = n * (acc.row_bytes("fp8") + acc.INDEX_BYTES)
    assert by - gathered == B * 16 * (576 + 512 * 2)
    step = gathered * g["layers_per_step"]
    assert abs(step / 1e9 - c["gb_per_step"]) < 0.05
    assert abs(step / g["peak_bytes_per_s"] * 1e3 - c["floor_ms_per_step"]) < 0.005
    assert abs(by * g["layers_per_step"] / g["peak_bytes_per_s"] * 1e3 - c["floor_ms_per_step"]) < 0.005


def test_generated_headline_shapes_match_captured_arguments(golden):
    g = golden("issue_arguments.json")["c16"]
    lengths = workloads.c16_lengths()
    assert len(lengths) == 16
    lo, hi, total = g["kv_len_min_max_sum_late"][0]
    assert (min(lengths), max(lengths)) == (lo, hi)
    assert abs(sum(lengths) - total) <= 2
    assert workloads.POOL_ENTRIES == g["kv_buffer"]["shape"][0]
    assert workloads.INDEX_BUFFER == g["kv_indices"]["shape"][0]


def test_c24_lengths_stay_in_captured_range(golden):
    g = golden("issue_arguments.json")["c24"]
    lengths = workloads.c24_lengths()
    assert len(lengths) == 24
    lo = min(r[0] for r in g["kv_len_min_max_sum_late"])
    hi = max(r[1] for r in g["kv_len_min_max_sum_late"])
    assert lo - 500 <= min(lengths) and max(lengths) <= hi


def test_cascade_bytes_count_the_shared_prefix_once():
    """Distinct slots of the batch-16 call: the 63,911-slot prefix once plus
    16 unique tails (the pages' "~137k distinct slots", 8.04x fewer)."""
    w = workloads.Workload(name="c16-lengths", dtype="fp8", q=None, kv_pool=None, qo_indptr=None,
                           kv_indptr=None, kv_indices=None, kv_last_page_lens=None, q_scale=None,
                           kv_scale=None, sm_scale=0.0, num_heads=16, real_heads=12,
                           max_seqlen_q=1, return_lse=False, lengths=workloads.c16_lengths(),
                           qlens=[1] * 16)
    P = workloads.SHARED_PREFIX
    distinct = P + sum(n - P for n in w.lengths)
    assert distinct == 63_911 + 16 * 4_519 + sum(b % 5 for b in range(16))
    assert acc.cascade_bytes(w, P) == distinct * 580 + 16 * 16 * (576 + 1024)
    assert abs(acc.workload_bytes(w) / acc.cascade_bytes(w, P) - 8.0) < 0.1
    assert acc.cascade_bytes(w, 0) == acc.workload_bytes(w)
