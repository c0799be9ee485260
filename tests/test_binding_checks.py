"""CPU checks of the Python binding's argument validation.

The C ABI receives pointers and strides only, so it cannot see how large a
buffer is or which dtype it holds. The binding checks every tensor's shape,
dtype and device against the layout the kernels address and raises
ValueError before it marshals anything. These tests use CPU tensors: a
mismatched argument is rejected by name; a consistent set gets as far as the
GPU-tensor check of the marshalling step. The library is replaced by a stub
that fails the test if any entry point is reached.
"""
import pytest
import torch

import context_causal_attention_cpattn_amd as cp

bf16, f32 = torch.bfloat16, torch.float32


class _NoLibrary:
    """Stands in for the loaded library: any entry point reached fails the test."""

    def __getattr__(self, name):
        def call(*args):
            pytest.fail(f"{name} was called")
        return call


@pytest.fixture(autouse=True)
def no_library(monkeypatch):
    monkeypatch.setattr(cp, "load", lambda: _NoLibrary())
B, H, Tq, Tk, D = 1, 2, 16, 24, 64
QMAP, KMAP = (Tq, Tq, 0, 0), (Tk, Tk, 0, 0)


def t(*shape, dtype=f32):
    return torch.zeros(*shape, dtype=dtype)


def fwd_args(**over):
    a = dict(q=t(B, H, Tq, D, dtype=bf16), k=t(B, H, Tk, D, dtype=bf16), v=t(B, H, Tk, D, dtype=bf16),
             qmap=QMAP, kmap=KMAP, o=t(B, H, Tq, D), lse=t(B, H, Tq))
    a.update(over)
    return a


def bwd_args(**over):
    a = dict(q=t(B, H, Tq, D, dtype=bf16), k=t(B, H, Tk, D, dtype=bf16), v=t(B, H, Tk, D, dtype=bf16),
             dout=t(B, H, Tq, D, dtype=bf16), lse=t(B, H, Tq), delta=t(B, H, Tq), dq_acc=t(B, H, Tq, D),
             dk_acc=t(B, H, Tk, D), dv_acc=t(B, H, Tk, D), qmap=QMAP, kmap=KMAP)
    a.update(over)
    return a


def test_block_fwd_consistent_set_reaches_marshalling():
    with pytest.raises(ValueError, match="GPU tensors"):
        cp.cpattn_block_fwd(**fwd_args())


@pytest.mark.parametrize("over,msg", [
    (dict(o=t(B, H, Tq, D, dtype=bf16)), "o: dtype"),
    (dict(k=t(B, H, Tk, D)), "k: dtype"),
    (dict(v=t(B, H, Tk - 1, D, dtype=bf16)), "v: shape"),
    (dict(lse=t(B, H, Tq - 1)), "lse: shape"),
    (dict(o=t(B, H, Tq, D // 2)), "o: shape"),
    (dict(k=t(B, H + 1, Tk, D, dtype=bf16)), "k has 3 heads"),
    (dict(q=t(B, H, Tq, D, dtype=torch.float16)), "unsupported dtype"),
])
def test_block_fwd_rejects_mismatched_tensors(over, msg):
    with pytest.raises(ValueError, match=msg):
        cp.cpattn_block_fwd(**fwd_args(**over))


def test_block_fwd_rejects_bad_rope_table():
    with pytest.raises(ValueError, match="rope_table: shape"):
        cp.cpattn_block_fwd(**fwd_args(), rope_table=t(64, D // 2))
    with pytest.raises(ValueError, match="rope_table: dtype"):
        cp.cpattn_block_fwd(**fwd_args(), rope_table=t(64, D, dtype=bf16))


def test_block_fwd_merge_and_gqa_check_accumulators():
    a = fwd_args(k=t(B, 1, Tk, D, dtype=bf16), v=t(B, 1, Tk, D, dtype=bf16))
    o, lse = a.pop("o"), a.pop("lse")
    with pytest.raises(ValueError, match="o_acc: dtype"):
        cp.cpattn_block_fwd_merge(**a, o_acc=o.to(bf16), lse_acc=lse)
    with pytest.raises(ValueError, match="lse_acc: shape"):
        cp.cpattn_block_fwd_merge(**a, o_acc=o, lse_acc=t(B, H, Tq + 1))
    with pytest.raises(ValueError, match="GPU tensors"):
        cp.cpattn_block_fwd_gqa(**a, o=o, lse=lse)


@pytest.mark.parametrize("fn", [cp.cpattn_block_bwd, cp.cpattn_block_bwd_gqa])
def test_block_bwd_consistent_set_reaches_marshalling(fn):
    with pytest.raises(ValueError, match="GPU tensors"):
        fn(**bwd_args())


@pytest.mark.parametrize("over,msg", [
    (dict(dk_acc=t(B, H, Tk, D, dtype=bf16)), "dk_acc: dtype"),   # zeros_like(k)
    (dict(dv_acc=t(B, H, Tk - 8, D)), "dv_acc: shape"),
    (dict(dq_acc=t(B, H, Tq, D, dtype=bf16)), "dq_acc: dtype"),
    (dict(dout=t(B, H, Tq, D)), "dout: dtype"),
    (dict(delta=t(B, H, Tq - 1)), "delta: shape"),
    (dict(lse=t(B, H, Tq, dtype=bf16)), "lse: dtype"),
    (dict(v=t(B, H, Tk, D)), "v: dtype"),
])
def test_block_bwd_rejects_mismatched_tensors(over, msg):
    with pytest.raises(ValueError, match=msg):
        cp.cpattn_block_bwd(**bwd_args(**over))


def test_block_bwd_halves_check_only_their_accumulators():
    a = bwd_args()
    dq = a.pop("dq_acc")
    with pytest.raises(ValueError, match="dv_acc: dtype"):
        cp.cpattn_block_bwd_dkdv(**dict(a, dv_acc=t(B, H, Tk, D, dtype=bf16)))
    a = bwd_args()
    a.pop("dk_acc"), a.pop("dv_acc")
    with pytest.raises(ValueError, match="dq_acc: shape"):
        cp.cpattn_block_bwd_dq(**dict(a, dq_acc=t(B, H, Tq - 1, D)))
    with pytest.raises(ValueError, match="GPU tensors"):
        cp.cpattn_block_bwd_dq(**dict(a, dq_acc=dq))


def test_gqa_bwd_accumulators_have_kv_heads():
    a = bwd_args(k=t(B, 1, Tk, D, dtype=bf16), v=t(B, 1, Tk, D, dtype=bf16))
    with pytest.raises(ValueError, match="dk_acc: shape"):
        cp.cpattn_block_bwd_gqa(**a)  # dk_acc still has H heads
    a.update(dk_acc=t(B, 1, Tk, D), dv_acc=t(B, 1, Tk, D))
    with pytest.raises(ValueError, match="GPU tensors"):
        cp.cpattn_block_bwd_gqa(**a)


def test_merge_preprocess_and_rotary_reject():
    o, l = t(B, H, Tq, D), t(B, H, Tq)
    with pytest.raises(ValueError, match="o_blk: shape"):
        cp.cpattn_lse_merge(o, l, t(B, H, Tq - 1, D), l)
    with pytest.raises(ValueError, match="lse_blk: dtype"):
        cp.cpattn_lse_merge(o, l, o, l.to(bf16))
    with pytest.raises(ValueError, match="o: dtype"):
        cp.cpattn_bwd_preprocess(t(B, H, Tq, D, dtype=bf16), o.to(bf16), l)
    with pytest.raises(ValueError, match="delta: shape"):
        cp.cpattn_bwd_preprocess(t(B, H, Tq, D, dtype=bf16), o, t(B, H, Tq + 1))
    x = t(B, H, Tq, D, dtype=bf16)
    with pytest.raises(ValueError, match="out: shape"):
        cp.cpattn_rope_rotate(x, QMAP, t(64, D), out=t(B, H, Tq - 1, D, dtype=bf16))
    with pytest.raises(ValueError, match="rope_table is required"):
        cp.cpattn_rope_rotate(x, QMAP, None)
    with pytest.raises(ValueError, match="g: dtype"):
        cp.cpattn_rope_rotate_grad(x, QMAP, t(64, D))


def test_ring_entry_points_check_every_block():
    q = t(B, H, Tq, D, dtype=bf16)
    kb = [t(B, H, Tq, D, dtype=bf16), t(B, H, Tq, D, dtype=bf16)]
    vb = [t(B, H, Tq, D, dtype=bf16), t(B, H, Tq - 1, D, dtype=bf16)]
    maps = [QMAP, QMAP]
    with pytest.raises(ValueError, match=r"v_blocks\[1\]: shape"):
        cp.cpattn_ring_fwd(q, kb, vb, maps, 0, QMAP, t(B, H, Tq, D), t(B, H, Tq), None)
    vb[1] = t(B, H, Tq, D, dtype=bf16)
    with pytest.raises(ValueError, match="o_acc: dtype"):
        cp.cpattn_ring_fwd(q, kb, vb, maps, 0, QMAP, t(B, H, Tq, D, dtype=bf16), t(B, H, Tq), None)
    dk = [t(B, H, Tq, D), t(B, H, Tq, D, dtype=bf16)]
    dv = [t(B, H, Tq, D), t(B, H, Tq, D)]
    with pytest.raises(ValueError, match=r"dk_blocks\[1\]: dtype"):
        cp.cpattn_ring_bwd(q, kb, vb, maps, 0, QMAP, q, t(B, H, Tq, D), t(B, H, Tq), t(B, H, Tq, D), dk, dv, None)
