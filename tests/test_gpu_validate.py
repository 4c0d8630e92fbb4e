"""Device-side validation (fd_set_validation / FD_VALIDATE=1): out-of-range
lengths and block-table entries are reported as FD_ERR_INVALID_ARG before
any attention kernel runs; valid calls give the same bits as without it."""

import numpy as np
import pytest
import torch

from tests.gpu_cases import to_dev, to_host
from workloads import synth

pytestmark = pytest.mark.gpu


@pytest.fixture
def validating(fd):
    fd.set_validation(True)
    yield fd
    fd.set_validation(False)


def test_validation_reports_bad_lengths(validating):
    fd = validating
    case = synth.decode_case(3, 16, 2, 128, 600, "bf16", seed=7700, lens=[600, 300, 1])
    q, k, v = (to_dev(case[x], "bf16") for x in ("q", "k", "v"))
    good = torch.from_numpy(case["lens"]).cuda()
    ref = fd.decode_attn(q, k, v, good, n_splits=4)
    fd.set_validation(False)
    plain = fd.decode_attn(q, k, v, good, n_splits=4)
    fd.set_validation(True)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(ref), to_host(plain))
    for bad in ([600, 0, 1], [601, 300, 1], [600, 300, -5]):
        with pytest.raises(fd.FdError) as e:
            fd.decode_attn(q, k, v, torch.tensor(bad, dtype=torch.int32, device="cuda"), n_splits=4)
        assert e.value.status == fd.FD_ERR_INVALID_ARG
        assert "FD_VALIDATE" in str(e.value)
    # bifurcated: dec_lens may be 0 but not above Ldmax
    c = synth.bifurcated_case(3, 8, 2, 128, 300, 16, "bf16", seed=7701, dec_lens=[16, 0, 5])
    t = {x: to_dev(c[x], "bf16") for x in ("q", "k_ctx", "v_ctx", "k_dec", "v_dec")}
    fd.bifurcated_attn(t["q"], t["k_ctx"], t["v_ctx"], t["k_dec"], t["v_dec"],
                       torch.from_numpy(c["dec_lens"]).cuda())
    with pytest.raises(fd.FdError) as e:
        fd.bifurcated_attn(t["q"], t["k_ctx"], t["v_ctx"], t["k_dec"], t["v_dec"],
                           torch.tensor([16, 17, 5], dtype=torch.int32, device="cuda"))
    assert e.value.status == fd.FD_ERR_INVALID_ARG


def test_validation_reports_bad_page_ids(validating):
    fd = validating
    case = synth.decode_case(2, 16, 2, 128, 300, "bf16", seed=7702, lens=[300, 40])
    kp, vp, table = synth.paginate(case["k"], case["v"], case["lens"], 16, seed=7702)
    q = to_dev(case["q"], "bf16")
    kpd, vpd = to_dev(kp, "bf16"), to_dev(vp, "bf16")
    lens = torch.from_numpy(case["lens"]).cuda()
    fd.decode_attn_paged(q, kpd, vpd, torch.from_numpy(table).cuda(), lens, n_splits=3)
    bad = table.copy()
    bad[1, 1] = kp.shape[0]          # a page id past the pool, in a block sequence 1 uses
    with pytest.raises(fd.FdError) as e:
        fd.decode_attn_paged(q, kpd, vpd, torch.from_numpy(bad).cuda(), lens, n_splits=3)
    assert e.value.status == fd.FD_ERR_INVALID_ARG
    unused = table.copy()
    unused[1, 5] = 10 ** 6           # past sequence 1's rows: never read, so accepted
    fd.decode_attn_paged(q, kpd, vpd, torch.from_numpy(unused).cuda(), lens, n_splits=3)
    torch.cuda.synchronize()
