"""The CPU oracle against its pins, and the pins against planted mistakes.

The second half copies the oracle's source, plants one plausible mistake (a
dropped term, a wrong sign or index, a transposed operand, an off-by-one) and
checks that at least one pin fails on the copy.  The mistakes live only in
in-memory copies; the oracle module itself is never modified.
"""
import inspect
import types

import pytest

import oracle.attention as oracle_mod
from tests import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(oracle_mod)


MUTATIONS = [
    ("scale_1_over_d", "return 1.0 / math.sqrt(head_dim)", "return 1.0 / head_dim"),
    ("exclusive_diagonal", "return k_pos[None, :] <= q_pos[:, None]",
     "return k_pos[None, :] < q_pos[:, None]"),
    ("gqa_modulo", "return h // (heads_q // heads_kv)", "return h % heads_kv"),
    ("striped_as_contiguous", "return i % p", "return i // (S // p)"),
    ("zigzag_wrong_tail", "np.where(sub < p, sub, 2 * p - 1 - sub)", "np.where(sub < p, sub, sub - p)"),
    ("ring_wrong_direction", "held[(r - 1) % world]", "held[(r + 1) % world]"),
    ("lse_drops_max", "np.where(live, m0 + np.log(zsafe), -np.inf)", "np.where(live, np.log(zsafe), -np.inf)"),
    ("output_unnormalised", "(e @ v) / zsafe[:, None]", "(e @ v)"),
    ("scale_dropped", "s = (q[a:b] @ k.T) * scale", "s = (q[a:b] @ k.T)"),
    ("key_prefix_off_by_one", "return int(q_pos_block.max()) + 1", "return int(q_pos_block.max())"),
    ("ds_sign", "dS = P * (dP - D[:, None])", "dS = P * (dP + D[:, None])"),
    ("dk_scale_dropped", "dK[bi, g, :lim] += (dS.T @ q) * scale", "dK[bi, g, :lim] += (dS.T @ q)"),
    ("dq_scale_dropped", "(dS @ k) * scale", "(dS @ k)"),
    ("dv_overwrites", "dV[bi, g, :lim] += P.T @ do", "dV[bi, g, :lim] = P.T @ do"),
    ("delta_drops_o", "D = np.sum(do * O, axis=1)", "D = np.sum(do, axis=1)"),
    ("bwd_unmasked", "s = np.where(_visible(key_pos[:lim], rb), s, -np.inf)", "s = s"),
    ("dq_uses_v", "(dS @ k) * scale", "(dS @ v) * scale"),
    ("merge_weights_swapped", "o = wa[..., None] * o_a + wb[..., None] * o_b",
     "o = wb[..., None] * o_a + wa[..., None] * o_b"),
    ("merge_lse_drops_max", "hi + np.log(wa_raw + wb_raw)", "np.log(wa_raw + wb_raw)"),
    ("delta_transposed", "axis=-1)", "axis=0)"),
    ("docs_ignored", "return (k_doc[None, :] == q_doc[:, None]) & (k_doc[None, :] >= 0)",
     "return (k_doc[None, :] >= 0) & (q_doc[:, None] >= 0)"),
    ("padding_keys_visible", "return (k_doc[None, :] == q_doc[:, None]) & (k_doc[None, :] >= 0)",
     "return k_doc[None, :] == q_doc[:, None]"),
    ("doc_boundary_off_by_one", "doc[e[k]:e[k + 1]] = k", "doc[e[k]:e[k + 1] + 1] = k"),
    ("padding_in_first_doc", "doc = np.full(S, -1, dtype=np.int64)", "doc = np.full(S, 0, dtype=np.int64)"),
    ("bwd_ignores_docs",
     "s = np.where(_same_document(docs[bi][:lim], docs[bi][rb]), s, -np.inf)", "s = s"),
    ("partial_ignores_docs", "qd, kd = docs[bi][q_pos], docs[bi][k_pos]", "qd, kd = None, None"),
]


def _mutant(old, new):
    src = inspect.getsource(oracle_mod)
    assert src.count(old) == 1, f"mutation anchor not unique: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    mod.__dict__["__name__"] = "oracle_mutant"
    exec(compile(src.replace(old, new), "<oracle_mutant>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(name, old, new):
    mod = _mutant(old, new)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(mod)
        except Exception as e:  # an assertion or a crash both count as caught
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin caught the planted mistake {name}"
