"""Host-side checks of bench.py (no GPU): the one-GPU contract, the workload table
and the paged workload's pools, which must hold the masked-cache workload's caches."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_workload_table():
    sys.path.insert(0, ROOT)
    import bench
    for name in ("layer_prefill_8b", "ffn_prefill_3b", "attn_prefill_8b", "layer_decode_8b",
                 "attn_decode_8b", "ffn_decode_8b_B1", "ffn_decode_8b_B64", "router_prefill_8b",
                 "attn_decode_masked_cache_8b", "attn_decode_paged_8b_p16",
                 "attn_decode_paged_8b_p128"):
        assert name in bench.WORKLOADS, name


def test_paged_workload_pools_hold_the_masked_cache():
    """Gathering the paged workload's pools through its table gives the masked-cache
    workload's caches (zero-padded to whole pages) and the same lengths."""
    sys.path.insert(0, ROOT)
    import bench
    from oracle import paged_to_contiguous
    w = bench.AttnDecodePaged(B=2, pos=300, page_size=16)
    c = w.c
    K, V, L = paged_to_contiguous(w._pool(c["K_cache"]), w._pool(c["V_cache"]), w.table, w.lens)
    cap = c["K_cache"].shape[2]
    assert np.array_equal(K[:, :, :cap], c["K_cache"]) and np.all(K[:, :, cap:] == 0)
    assert np.array_equal(V[:, :, :cap], c["V_cache"])
    assert np.array_equal(L, w.lens)
    assert sorted(w.table.reshape(-1).tolist()) == list(range(w.n_pages))  # a permutation
