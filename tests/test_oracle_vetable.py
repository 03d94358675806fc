"""Pins of the value-embedding table lookup and its gradient: torch's embedding lookup and
its autograd in float64 (a library routine), and the hand-evaluated accumulation of repeated
ids. CPU only."""

import numpy as np
import torch
import torch.nn.functional as F

import oracle


def test_lookup_matches_torch_embedding():
    rng = np.random.default_rng(1)
    table = rng.standard_normal((50, 24))
    ids = rng.integers(0, 50, (3, 17))
    np.testing.assert_array_equal(oracle.ve_lookup(table, ids),
                                  F.embedding(torch.from_numpy(ids), torch.from_numpy(table)).numpy())


def test_invalid_ids_give_zero_rows_and_no_gradient():
    table = np.arange(12.0).reshape(3, 4)
    ids = np.array([[0, -1, 2, 3]])
    out = oracle.ve_lookup(table, ids)
    np.testing.assert_array_equal(out[0, 1], 0.0)
    np.testing.assert_array_equal(out[0, 3], 0.0)
    g = oracle.ve_table_grad(np.ones((1, 4, 4)), ids, 3)
    np.testing.assert_array_equal(g, [[1.0] * 4, [0.0] * 4, [1.0] * 4])


def test_table_gradient_matches_torch_autograd():
    rng = np.random.default_rng(2)
    table = torch.from_numpy(rng.standard_normal((40, 16))).requires_grad_(True)
    ids = torch.from_numpy(rng.integers(0, 40, (4, 30)))      # repeats on purpose
    dve = rng.standard_normal((4, 30, 16))
    F.embedding(ids, table).backward(torch.from_numpy(dve))
    np.testing.assert_allclose(oracle.ve_table_grad(dve, ids.numpy(), 40), table.grad.numpy(),
                               rtol=1e-13, atol=1e-13)


def test_repeated_ids_accumulate():
    dve = np.array([[[1.0, 2.0], [10.0, 20.0], [100.0, 200.0]]])
    np.testing.assert_array_equal(oracle.ve_table_grad(dve, np.array([[1, 1, 0]]), 2),
                                  [[100.0, 200.0], [11.0, 22.0]])
