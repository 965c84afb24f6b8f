"""The checked build (libmoeffn_checked.so: bounds tests on every index a
call produces for itself -- prefill row lists and slot positions, decode
routing plans -- reported through MOE_FLAG_CHECK) on the same inputs as the
default build: no test fails and the outputs are bitwise the same, on the
decode and prefill paths, both weight formats' tiles and the wrapper.
Needs an MI355X; run with ``-m gpu``."""

from __future__ import annotations

import numpy as np
import pytest

from mixture_experts_ffn_rmsnorm_amd import inputs as gen
from mixture_experts_ffn_rmsnorm_amd import moe
from oracle import moe_ref as ref
from tests.gpu_common import Layer

pytestmark = [pytest.mark.gpu, pytest.mark.filterwarnings("ignore::RuntimeWarning")]

SCORE, HASH = ref.LAYER_SCORE, ref.LAYER_HASH


def _both(run):
    """run() under the default and the checked build."""
    a = run()
    with moe.using(moe.CHECKED_LIB_PATH):
        b = run()
    return a, b


def _same(a, b, what):
    out_a, st_a = a
    out_b, st_b = b
    assert st_a == 0 and st_b == 0, f"{what}: status {st_a} / {st_b}"
    np.testing.assert_array_equal(out_a, out_b, err_msg=what)


@pytest.fixture(scope="module")
def tiny():
    return Layer(gen.config(0))


@pytest.mark.parametrize("rows", [1, 3, 4, 37, 300])
@pytest.mark.parametrize("kind", [SCORE, HASH])
def test_tiny_checked_equals_default(tiny, rows, kind):
    x = np.random.default_rng(600 + rows).standard_normal((rows, tiny.cfg.hidden)).astype(np.float32)
    tok = np.random.default_rng(610 + rows).integers(0, tiny.cfg.table_rows, rows).astype(np.int32)
    a, b = _both(lambda: tuple(tiny.run(x, tok if kind == HASH else None, kind)[i] for i in (0, 4)))
    _same(a, b, f"tiny rows={rows} kind={kind}")


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
@pytest.mark.parametrize("rows", [2, 37, 300])
def test_tiny_mx_checked_equals_default(fmt, rows):
    from tests.test_gpu_mx import MxLayer

    lay = MxLayer(gen.config(0), fmt=fmt)
    x = np.random.default_rng(620 + rows).standard_normal((rows, lay.cfg.hidden)).astype(np.float32)
    a, b = _both(lambda: tuple(lay.run(x, None, SCORE)[i] for i in (0, 4)))
    _same(a, b, f"{fmt} rows={rows}")


@pytest.mark.parametrize("rows", [1, 4, 37])
def test_tiny_hc_checked_equals_default(tiny, rows):
    from tests.test_gpu_hc import HcLayer

    hl = HcLayer(tiny, 4, rows)
    a, b = _both(lambda: (lambda g: (g["out"], g["status"]))(hl.run(hl.host.state, None, SCORE)))
    _same(a, b, f"hc rows={rows}")


def test_full_checked_equals_default():
    """The full shape: one row, the 4-row cohort and 512 rows."""
    full = Layer(gen.config(1))
    for cfg_i, kind in ((1, SCORE), (2, HASH), (3, SCORE)):
        cfg = gen.config(cfg_i)
        lay = full if cfg_i == 1 else Layer(cfg, share=full)
        hi = lay.host
        tok = hi.token_ids if kind == HASH else None
        a, b = _both(lambda: tuple(lay.run(hi.x, tok, kind)[i] for i in (0, 4)))
        _same(a, b, cfg.name)
