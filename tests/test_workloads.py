"""Host checks of the seeded workload generators (CPU only)."""
import numpy as np

from paged_quantized_kv_ra_amd import workloads as W


def test_deterministic():
    a, b = W.tiny_decode(), W.tiny_decode()
    assert np.array_equal(a.q, b.q) and np.array_equal(a.tokens_k, b.tokens_k)
    assert np.array_equal(a.block_tables, b.block_tables)


def test_tiny_decode_shape():
    w = W.tiny_decode()
    assert w.batch == 1 and w.ctx[0] == 256 and w.num_pages == 32
    row = w.block_tables[0, :16]
    assert len(set(row.tolist())) == 16 and row.max() < 32
    assert w.block_tables[0, 16] == W.INT32_MAX
    assert w.q.dtype == np.float16 and w.q.shape == (1, 4, 64)
    assert abs(w.softmax_scale - 0.125) < 1e-15


def test_batch8_contexts_and_pages():
    w = W.batch8_decode()
    assert np.all((w.ctx >= 1024) & (w.ctx <= 8192))
    used = np.concatenate([w.block_tables[b, :-(-int(w.ctx[b]) // 16)] for b in range(8)])
    assert len(np.unique(used)) == used.size and used.max() < 8192
    assert w.q.dtype == np.uint16  # bf16 bit patterns


def test_slots_match_block_tables():
    w = W.build("t", 0, ctx=[50, 33, 70], q_len=[3, 1, 5], num_q_heads=4,
                num_kv_heads=2, head_dim=64, kv_dtype="e4m3", pool_pages=20,
                shared_prefix_tokens=32)
    for b in range(w.batch):
        rows = w.seq_rows[b]
        j = np.arange(int(w.ctx[b]))
        want = w.block_tables[b, j // 16].astype(np.int64) * 16 + j % 16
        assert np.array_equal(w.token_slots[rows], want)
    # the shared prefix maps to the same rows and pages in every sequence
    assert np.array_equal(w.seq_rows[0][:32], w.seq_rows[2][:32])
    assert np.array_equal(w.block_tables[0, :2], w.block_tables[1, :2])
    assert w.new_token_rows().shape == (9,)
    assert w.k_scale > 0 and w.v_scale > 0


def test_attended_keys_window():
    w = W.build("t", 0, ctx=[1000, 30], q_len=[16, 4], num_q_heads=4, num_kv_heads=2,
                head_dim=64, kv_dtype="e4m3", window_left=100, num_sinks=4)
    # seq 0: window covers [1000-16-100+1, 1000) = 115 keys, plus 4 sinks
    # seq 1: window reaches position 0, sinks add nothing
    assert w.attended_keys() == 115 + 4 + 30
