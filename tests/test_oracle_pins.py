"""The oracle against its pins (closed forms, worked examples, textbook routines, invariants)."""
import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_oracle_rejects_bad_arguments(orc):
    import numpy as np

    q = np.zeros((4, 1, 2))
    with pytest.raises(ValueError):
        orc.quadratic(q, q, q, np.ones(1), cu_seqlens=np.array([0, 3], np.int32))  # cu[S] != T
    with pytest.raises(ValueError):
        orc.quadratic(q, q, q, np.ones(1), cu_seqlens=np.array([0, 3, 2, 4], np.int32))
    with pytest.raises(ValueError):
        orc.quadratic_rows(q, q, q, np.ones(1), [4])


def test_oracle_regression_fixture(orc):
    """The oracle still reproduces the outputs it wrote to tests/golden/oracle_regression.json."""
    import json
    import os

    import numpy as np

    from golden.make_golden import case

    path = os.path.join(os.path.dirname(__file__), "golden", "oracle_regression.json")
    doc = json.load(open(path))
    q, k, v, lam, cu, S0 = case()
    out = orc.quadratic(q, k, v, lam, cu, init_state=S0)
    st = orc.final_state(k, v, lam, cu, init_state=S0)
    assert np.allclose(out, np.array(doc["out"]), rtol=1e-13, atol=1e-13)
    assert np.allclose(st, np.array(doc["final_state"]), rtol=1e-13, atol=1e-13)


def test_oracle_backward_regression_fixture(orc):
    """The backward oracle still reproduces the gradients stored in the same fixture."""
    import json
    import os

    import numpy as np

    from golden.make_golden import backward_case

    doc = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                      "oracle_regression.json")))
    q, k, v, lam, cu, S0, d_out, d_final = backward_case()
    got = orc.backward(q, k, v, lam, d_out, cu, init_state=S0, d_final=d_final)
    for name, g in zip(("dq", "dk", "dv", "d_init"), got):
        assert np.allclose(g, np.array(doc[name]), rtol=1e-13, atol=1e-13), name
