"""CPU checks of the test harness that runs the oracle in token blocks, and
of the per-slot exact integer reference used at full workload sizes."""
import numpy as np

import synth
from tests import bounds, oracle_par


def test_linear_blocks_equal_whole_batch(oracle_mod):
    c = synth.config_decode(T=97)
    whole, _ = oracle_mod.lora_apply(c.y0, c.x, c.A, c.B, c.idx, c.slot_rank, c.scale)
    for threads in (1, 3, 8):
        got = oracle_par.lora_apply(oracle_mod, c.y0, c.x, c.A, c.B, c.idx, c.slot_rank, c.scale,
                                    threads=threads)
        assert np.array_equal(got.view(np.uint32), whole.view(np.uint32))
    rows = np.array([0, 5, 96, 40])
    sub = oracle_par.lora_apply(oracle_mod, c.y0, c.x, c.A, c.B, c.idx, c.slot_rank, c.scale,
                                threads=2, rows=rows)
    assert np.array_equal(sub, whole[rows])


def test_moe_blocks_equal_whole_batch(oracle_mod):
    c = synth.make_moe("par", 37, 4, 8, 128, 64, 16, 3, "bf16", 3)
    w13 = oracle_mod.moe_lora_apply(0, c.gate_up0, c.x, c.A13, c.B13, c.topk_ids, None, c.idx,
                                    c.slot_rank, c.scale, c.E)
    got = oracle_par.moe_lora_apply(oracle_mod, 0, c.gate_up0, c.x, c.A13, c.B13, c.topk_ids,
                                    None, c.idx, c.slot_rank, c.scale, c.E, threads=5)
    assert np.array_equal(got, w13)
    w2 = oracle_mod.moe_lora_apply(1, c.out0, c.h, [c.A2], [c.B2], c.topk_ids, c.topk_w, c.idx,
                                   c.slot_rank, c.scale, c.E)
    got = oracle_par.moe_lora_apply(oracle_mod, 1, c.out0, c.h, [c.A2], [c.B2], c.topk_ids,
                                    c.topk_w, c.idx, c.slot_rank, c.scale, c.E, threads=4)
    assert np.array_equal(got, w2)
    z = np.zeros((c.T, c.K), np.float32)
    red = oracle_mod.moe_lora_apply(1, z, c.h, [c.A2], [c.B2], c.topk_ids, c.topk_w, c.idx,
                                    c.slot_rank, c.scale, c.E, reduce_k=True)
    got = oracle_par.moe_lora_apply(oracle_mod, 1, z, c.h, [c.A2], [c.B2], c.topk_ids, c.topk_w,
                                    c.idx, c.slot_rank, c.scale, c.E, reduce_k=True, threads=3)
    assert np.array_equal(got, red)


def test_exact_int_by_slot_equals_int64():
    c = synth.make_integer_linear(120, 256, [64, 40], 16, 5, seed=3)
    a = bounds.linear_exact_int(c.x, c.A, c.B, c.idx, c.slot_rank, c.scale, c.y0)
    b = bounds.linear_exact_int_by_slot(c.x, c.A, c.B, c.idx, c.slot_rank, c.scale, c.y0)
    assert np.array_equal(a.astype(np.float64), b)


def test_ternary_rows_have_the_stated_non_zeros():
    rng = np.random.default_rng(1)
    a = synth.ternary_sparse(rng, (4, 7, 300), 32)
    assert set(np.unique(a)) <= {-1.0, 0.0, 1.0}
    assert np.all(np.count_nonzero(a, axis=-1) == 32)
    b = synth.ternary_sparse(rng, (3, 5), 9)        # fewer columns than non-zeros
    assert np.all(np.abs(b) == 1.0)
