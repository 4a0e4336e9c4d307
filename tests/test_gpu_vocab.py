"""GPU parity of the vocabulary-sized variants against the fp64 oracle:
the LM-head logits delta (vLLM punica_base.py, add_lora_logits: the shrink
and expand with the sampled rows' adapters, N = the vocabulary) and the
embedding delta (add_lora_embedding: the expand alone, y += x @ B)."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from tenant_lora_serving_amd import inputs as I
from tenant_lora_serving_amd import lora as B
from gpu_util import assert_close, assert_close_chunked, assert_ws_ok, bf64, d16, d32, h16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def logits_case():
    # 256 sampled rows of a Llama-3-8B-class LM head: hidden 4096, vocabulary 128256
    return I.make_dense(41, n=256, k_in=4096, slice_sizes=(128256,), num_slots=32, max_rank=16,
                        rank_choices=[8, 16], slot_kind="zipf", neg_frac=0.05, scale_num=32.0)


def test_logits_full_vocab(logits_case):
    c = logits_case
    print(f"logits n={c.n} vocab={c.n_out}", flush=True)
    y = d16(c.y)
    ws = B.fused_workspace(c.n, c.num_slots, 1, c.max_rank, c.k_in)
    B.add_lora_logits(y, d16(c.x), d16(c.a_pool), d16(c.b_pool), d32(c.scale), d32(c.slot), ws=ws)
    assert_ws_ok(ws, calls=1)
    out = h16(y)
    act = (c.slot >= 0) & (c.slot < c.num_slots)
    assert np.array_equal(out[~act], c.y[~act])
    assert_close_chunked(out, lambda r: O.case_fused_rows(c, r), np.flatnonzero(act), "logits", chunk=32)


def test_logits_small_ragged():
    # a vocabulary that is not a multiple of 512: ragged last column batch
    c = I.make_dense(42, n=37, k_in=264, slice_sizes=(32008,), num_slots=5, max_rank=8,
                     slot_kind="uniform_neg")
    y = d16(c.y)
    ws = B.fused_workspace(c.n, c.num_slots, 1, c.max_rank, c.k_in)
    B.add_lora_logits(y, d16(c.x), d16(c.a_pool), d16(c.b_pool), d32(c.scale), d32(c.slot), ws=ws)
    assert_ws_ok(ws, calls=1)
    assert_close(bf64(h16(y)), O.case_fused_rows(c, np.arange(c.n)), "logits small")


@pytest.mark.parametrize("add_inputs", [True, False])
def test_embedding_expand(add_inputs):
    c = I.make_dense(43, n=512, k_in=64, slice_sizes=(4096,), num_slots=8, max_rank=16,
                     slot_kind="uniform_neg")
    xe = np.random.default_rng(43).standard_normal((c.n, c.max_rank)).astype(np.float32)
    y = d16(c.y)
    B.add_lora_embedding(y, d32(xe), d16(c.b_pool), d32(c.slot), add_inputs=add_inputs)
    torch.cuda.synchronize()
    out = h16(y)
    act = (c.slot >= 0) & (c.slot < c.num_slots)
    rows = np.flatnonzero(act)
    orc = O.expand_rows(xe[rows][:, None, :], c.b_pool, c.num_slots, (4096,), c.max_rank, c.slot, rows,
                        c.y, add_inputs=add_inputs)
    assert_close(bf64(out[rows]), orc, f"embedding add_inputs={add_inputs}")
    assert np.array_equal(out[~act], c.y[~act])
