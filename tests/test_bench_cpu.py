"""CPU checks of bench.py's accounting: the algorithmic bytes of a decode pass
and the algorithmic flops of a prefill call, against sums written out here from
the model's tensor shapes."""
import bench
import synth


def _block_matrix_elems(E):
    # qkv [E][3E], attention projection [E][E], fc [E][4E], MLP projection [4E][E]
    return 3 * E * E + E * E + 4 * E * E + 4 * E * E


def test_decode_bytes_fp32_124m():
    cfg = synth.CONFIGS[2]
    E, V, L, P = 768, 50257, 12, 1024
    small_per_layer = (2 * E) + (3 * E) + E + (2 * E) + 4 * E + E   # LN1, b_qkv, b_ap, LN2, b_fc, b_pr
    weights = 4 * (L * _block_matrix_elems(E) + V * E + L * small_per_layer + 2 * E)
    embed_rows = 2 * E * 4
    for p in (0, 1, 68, 1023):
        kv = L * 2 * E * 4 * (p + 1)   # K and V rows 0..p of every layer
        assert bench.bytes_per_step(cfg, p) == weights + embed_rows + kv
    # a 69-pass launch of the 10 + 60 workload
    assert sum(bench.bytes_per_step(cfg, p) for p in range(cfg.n_steps)) == 34_306_808_832


def test_decode_bytes_quantised():
    E, V, L = 768, 50257, 12
    f16, q4 = synth.CONFIGS[3], synth.CONFIGS[4]
    d32 = bench.bytes_per_step(synth.CONFIGS[2], 0)
    mats = L * _block_matrix_elems(E)
    # fp16: matrices and the head at 2 bytes
    assert d32 - bench.bytes_per_step(f16, 0) == 2 * mats + 2 * V * E
    # int4: half a byte per weight plus (scale, zero) float pairs per group of 32; fp32 head
    assert d32 - bench.bytes_per_step(q4, 0) == 4 * mats - (mats // 2 + mats // 32 * 8)


def test_prefill_flops():
    cfg = synth.CONFIGS[2]
    E, V, L = 768, 50257, 12
    # one row: the linears once, attention over one key, the head
    assert bench.prefill_flops(cfg, 1) == 2 * L * _block_matrix_elems(E) + L * 4 * E + 2 * V * E
    # n rows from position p0: row t attends to p0 + t + 1 keys
    n, p0 = 1024, 0
    keys = n * (n + 1) // 2
    assert bench.prefill_flops(cfg, n, p0) == 2 * n * L * _block_matrix_elems(E) + L * 4 * E * keys + 2 * V * E
    assert bench.prefill_flops(cfg, 10, 5) - bench.prefill_flops(cfg, 10, 0) == L * 4 * E * 5 * 10
