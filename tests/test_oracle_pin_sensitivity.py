"""Plant plausible mistakes in the oracle (on the CPU only) and check that the
pins catch each one.  This shows the pins constrain the oracle rather than
restate it."""
import math

import numpy as np
import pytest
from scipy.special import erf

import test_oracle_layout as TL
import test_oracle_mlp as TM
import test_oracle_reduce as TR
from oracle import layout as L
from oracle import mlp as O
from oracle import reduce as R


def _fails(fn, *args):
    try:
        fn(*args)
    except (AssertionError, ValueError, IndexError, pytest.fail.Exception):
        return True
    return False


def test_gelu_dropped_term(monkeypatch):
    monkeypatch.setattr(O, "gelu", lambda x: 0.5 * np.asarray(x, float) * erf(np.asarray(x, float) / math.sqrt(2)))
    assert _fails(TM.test_gelu_closed_forms)


def test_gelu_wrong_sign(monkeypatch):
    monkeypatch.setattr(O, "gelu", lambda x: 0.5 * np.asarray(x, float) * (1 - erf(np.asarray(x, float) / math.sqrt(2))))
    assert _fails(TM.test_brute_force_tiny_shapes, O.GELU_ERF)


def test_gelu_wrong_scale(monkeypatch):
    monkeypatch.setattr(O, "gelu", lambda x: 0.5 * np.asarray(x, float) * (1 + erf(np.asarray(x, float))))
    assert _fails(TM.test_gelu_closed_forms)


def test_mlp_transposed_second_operand(monkeypatch):
    real = O.mlp_rank

    def bad(X, A_i, B_i, act=O.GELU_ERF):
        x, a, b = O._f64(X), O._f64(A_i), O._f64(B_i)
        y = x @ a
        y = O.gelu(y) if act == O.GELU_ERF else y
        return y @ b.T if b.shape[0] == b.shape[1] else y @ b
    monkeypatch.setattr(O, "mlp_rank", bad)
    assert _fails(TM.test_brute_force_tiny_shapes, O.GELU_NONE)
    monkeypatch.setattr(O, "mlp_rank", real)


def test_mlp_activation_after_second_gemm(monkeypatch):
    def bad(X, A_i, B_i, act=O.GELU_ERF):
        z = O._f64(X) @ O._f64(A_i) @ O._f64(B_i)
        return O.gelu(z) if act == O.GELU_ERF else z
    monkeypatch.setattr(O, "mlp_rank", bad)
    assert _fails(TM.test_brute_force_tiny_shapes, O.GELU_ERF)


def test_split_inner_axis_outermost(monkeypatch):
    real = L.shard_boxes

    def bad(shape, spec):
        boxes, groups = real(shape, spec)
        m = len(spec.get("sharded_dim", []))
        if m == 2:  # enumerate b-outer / a-inner instead
            n0 = spec["sharded_dim"][0].get("num_shards") or spec["sharded_dim"][0]["simple_sharding"][0]["num_shards"]
            n1 = len(boxes) // n0
            boxes = [boxes[s0 * n1 + s1] for s1 in range(n1) for s0 in range(n0)]
        return boxes, groups
    monkeypatch.setattr(L, "shard_boxes", bad)
    case = [c for c in TL._load()["cases"] if c["name"] == "E3_both_axes"][0]
    assert _fails(TL.test_page_examples, case)


def test_split_device_keys_swapped(monkeypatch):
    real = L.expand_devices
    monkeypatch.setattr(L, "expand_devices", lambda spec: list(reversed(real(spec))))
    case = [c for c in TL._load()["cases"] if c["name"] == "E5_mixed_split_broadcast"][0]
    assert _fails(TL.test_page_examples, case)


def test_split_off_by_one_width(monkeypatch):
    real = L.shard_boxes

    def bad(shape, spec):
        boxes, groups = real(shape, spec)
        return [tuple((a, b) if b - a == s else (a, min(b + 1, s)) for (a, b), s in zip(box, shape))
                for box in boxes], groups
    monkeypatch.setattr(L, "shard_boxes", bad)
    assert _fails(TL.test_brute_force_against_inverse_formula, False)


def test_mesh_wrong_dim_used(monkeypatch):
    real = L.split_dims_mapping

    def bad(tensor, mesh_dims, process_ids, dims_mapping):
        q = len(mesh_dims)
        return real(tensor, mesh_dims, process_ids, [(q - 1 - j) if j >= 0 else j for j in dims_mapping])
    monkeypatch.setattr(L, "split_dims_mapping", bad)
    case = TL._load()["mesh_cases"][0]
    assert _fails(TL.test_page_2d_sbp_example, case)


def test_reduce_drops_last_partial(monkeypatch):
    real = R.reduce_full
    monkeypatch.setattr(R, "reduce_full", lambda parts: real(list(parts)[:-1]) if len(parts) > 1 else real(parts))
    assert _fails(TR.test_integer_partials_exact)


def test_reduce_split_wrong_block(monkeypatch):
    real = R.reduce_split
    monkeypatch.setattr(R, "reduce_split", lambda parts, s: list(reversed(real(parts, s))))
    assert _fails(TR.test_split_blocks_concatenate_to_full)


# ---- backward --------------------------------------------------------------

import test_oracle_backward as TB  # noqa: E402


def test_gelu_deriv_missing_density_term(monkeypatch):
    monkeypatch.setattr(O, "gelu_deriv", lambda x: 0.5 * (1 + erf(np.asarray(x, float) / math.sqrt(2))))
    assert _fails(TB.test_gelu_deriv_closed_forms)
    assert _fails(TB.test_backward_matches_finite_differences, O.GELU_ERF, 3, 4, 5)


def test_gelu_deriv_wrong_sign(monkeypatch):
    real = O.gelu_deriv
    monkeypatch.setattr(O, "gelu_deriv", lambda x: real(-np.asarray(x, float)))
    assert _fails(TB.test_gelu_deriv_matches_finite_difference)


def test_backward_skips_activation_derivative(monkeypatch):
    def bad(X, A_i, B_i, dZ, act=O.GELU_ERF):
        x, a, b, dz = O._f64(X), O._f64(A_i), O._f64(B_i), O._f64(dZ)
        h = x @ a
        y = O.gelu(h) if act == O.GELU_ERF else h
        dh = dz @ b.T
        return {"dH": dh, "dX_i": dh @ a.T, "dA_i": x.T @ dh, "dB_i": y.T @ dz}
    monkeypatch.setattr(O, "backward_rank", bad)
    assert _fails(TB.test_backward_matches_finite_differences, O.GELU_ERF, 3, 4, 5)


def test_backward_weight_gradient_uses_pre_activation(monkeypatch):
    real = O.backward_rank

    def bad(X, A_i, B_i, dZ, act=O.GELU_ERF):
        g = real(X, A_i, B_i, dZ, act)
        g["dB_i"] = (O._f64(X) @ O._f64(A_i)).T @ O._f64(dZ)   # H instead of Y = act(H)
        return g
    monkeypatch.setattr(O, "backward_rank", bad)
    assert _fails(TB.test_backward_matches_finite_differences, O.GELU_ERF, 3, 4, 5)


def test_backward_rank_sum_drops_a_rank(monkeypatch):
    real = O.backward_all_ranks

    def bad(X, A_shards, B_shards, dZ, act=O.GELU_ERF):
        return real(X, A_shards[:-1], B_shards[:-1], dZ, act)[0], *real(X, A_shards, B_shards, dZ, act)[1:]
    monkeypatch.setattr(O, "backward_all_ranks", bad)
    assert _fails(TB.test_sum_of_rank_gradients_is_the_unsharded_gradient, 3)


# ---- partial max / min, bias -------------------------------------------------

def test_reduce_max_as_min(monkeypatch):
    real = R.reduce_full

    def bad(parts, op="sum", bias=None):
        return real(parts, {"max": "min", "min": "max"}.get(op, op), bias)
    monkeypatch.setattr(R, "reduce_full", bad)
    assert _fails(TR.test_max_min_brute_force)


def test_bias_added_per_partial(monkeypatch):
    real = R.reduce_full

    def bad(parts, op="sum", bias=None):
        if bias is None:
            return real(parts, op)
        return real([np.asarray(p) + np.asarray(bias) for p in parts], op)
    monkeypatch.setattr(R, "reduce_full", bad)
    assert _fails(TR.test_bias_is_added_once_after_the_sum)


def test_gather_takes_last_replica(monkeypatch):
    import test_oracle_gather as TG

    def bad(pieces, shape, spec):
        boxes, groups = L.shard_boxes(shape, spec)
        out = np.zeros(tuple(shape))
        for box, grp in zip(boxes, groups):
            out[tuple(slice(a, b) for a, b in box)] = pieces[grp[-1]]
        return out
    monkeypatch.setattr(L, "gather", bad)
    assert _fails(TG.test_replica_taken_from_first_listed_device)


def test_gather_pieces_in_reverse_boxes(monkeypatch):
    import test_oracle_gather as TG
    real = L.shard_boxes

    def bad_gather(pieces, shape, spec):
        boxes, groups = real(shape, spec)
        out = np.zeros(tuple(shape), dtype=np.float32)
        for box, grp in zip(reversed(boxes), groups):
            out[tuple(slice(a, b) for a, b in box)] = pieces[grp[0]]
        return out
    monkeypatch.setattr(L, "gather", bad_gather)
    case = [c for c in TL._load()["cases"] if c["name"] == "E1_axis0"][0]
    assert _fails(TG.test_page_examples_gather_back, case)


def test_gather_dims_mapping_later_replica_overwrites(monkeypatch):
    import itertools
    import test_oracle_gather as TG

    def bad(pieces, shape, mesh_dims, process_ids, dims_mapping):
        out = np.zeros(tuple(shape))
        for linear, coord in enumerate(itertools.product(*[range(m) for m in mesh_dims])):
            sl = []
            for i, j in enumerate(dims_mapping):
                w = shape[i] // mesh_dims[j] if j >= 0 else shape[i]
                sl.append(slice(coord[j] * w, coord[j] * w + w) if j >= 0 else slice(0, shape[i]))
            out[tuple(sl)] = pieces[process_ids[linear]]
        return out
    monkeypatch.setattr(L, "gather_dims_mapping", bad)
    assert _fails(TG.test_replica_taken_from_first_listed_device)


def test_checker_union_instead_of_intersection(monkeypatch):
    import test_oracle_checker as TK
    from oracle import checker as K
    real = K.broadcast_binary

    def bad(shape1, spec1, shape2, spec2):
        out_shape, shards = real(shape1, spec1, shape2, spec2)
        every = sorted({d for _, devs in shards for d in devs})
        return out_shape, [(box, every) for box, _ in shards]
    monkeypatch.setattr(K, "broadcast_binary", bad)
    assert _fails(TK.test_page_composition_example)


def test_checker_merge_ignores_conflict(monkeypatch):
    import test_oracle_checker as TK
    from oracle import checker as K

    def bad(x_map, y_map, mesh_ndim):
        k = x_map[-1] if x_map[-1] >= 0 else y_map[-2]
        return list(x_map[:-1]) + [y_map[-1]], ([k] if k >= 0 else [])
    monkeypatch.setattr(K, "matmul_dims_mapping", bad)
    assert _fails(TK.test_matmul_rejections, [0, 1], [0, -1], "spec")


def test_checker_drops_partial(monkeypatch):
    import test_oracle_checker as TK
    from oracle import checker as K
    real = K.matmul_dims_mapping
    monkeypatch.setattr(K, "matmul_dims_mapping", lambda x, y, q: (real(x, y, q)[0], []))
    assert _fails(TK.test_brute_force_matmul_local_products, [2, 2])


def test_round_bf16_truncates(monkeypatch):
    import test_oracle_stack as TS

    def bad(x):
        x = np.asarray(x, dtype=np.float64)
        m, e = np.frexp(x)
        return np.ldexp(np.trunc(m * 256.0) / 256.0, e)
    monkeypatch.setattr(O, "round_bf16", bad)
    assert _fails(TS.test_round_bf16_hand_worked, 259.0, 260.0)


def test_stack_drops_bias_from_next_input(monkeypatch):
    import test_oracle_stack as TS

    def bad(X, layers, dtype="bf16"):
        x = O._f64(X)
        out = []
        for layer in layers:
            z = O.mlp_rank(x, layer["A_i"], layer["B_i"], layer.get("act", O.GELU_ERF))
            for p in layer.get("peers", []):
                z = z + O._f64(p)
            x = O.round_to(z, dtype)
            if layer.get("bias") is not None:
                z = z + O._f64(layer["bias"])[None, :]
            out.append((z, x))
        return out
    monkeypatch.setattr(O, "mlp_stack", bad)
    assert _fails(TS.test_sharded_stack_is_the_unsharded_network, O.GELU_NONE)
