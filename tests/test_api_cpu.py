"""The allocating compute_* calls without a GPU: they exist with the pages'
names and refuse host tensors (there is no CPU path)."""
import pytest
import torch

from linear_recurrence_scan_coefficient_amd import api


def test_names_follow_the_pages():
    """The seven compute_* names of the README's Kernels table, plus the
    grouped-launch block."""
    assert sorted(api.__all__) == sorted([
        "compute_gae", "compute_vtrace", "compute_retrace", "compute_lambda_returns",
        "compute_discounted_returns", "compute_eligibility_traces",
        "compute_episodic_prefix_sum", "grouped"])


def test_empty_grouped_block_launches_nothing():
    with api.grouped() as g:
        assert g.calls == []
    with pytest.raises(RuntimeError):  # an exception inside the block skips the launch
        with api.grouped() as g:
            raise RuntimeError("inside")


@pytest.mark.parametrize("fn,args", [
    (api.compute_gae, (torch.zeros(2, 3), torch.zeros(2, 3), torch.zeros(2, 3))),
    (api.compute_lambda_returns, (torch.zeros(2, 3), torch.zeros(2, 3), torch.zeros(2, 3))),
    (api.compute_discounted_returns, (torch.zeros(2, 3), torch.zeros(2, 3))),
    (api.compute_vtrace, (torch.zeros(2, 3),) * 4),
    (api.compute_eligibility_traces, (torch.zeros(2, 3), torch.zeros(2, 3))),
    (api.compute_episodic_prefix_sum, (torch.zeros(2, 3, dtype=torch.int32),
                                       torch.zeros(2, 3))),
    (api.compute_retrace, (torch.zeros(2, 3), torch.zeros(2, 3, 4), torch.zeros(2, 3, 4),
                           torch.zeros(2, 3, dtype=torch.int32), torch.ones(2, 3),
                           torch.zeros(2, 3), torch.zeros(2, 3))),
])
def test_host_tensors_are_refused(fn, args):
    with pytest.raises(ValueError, match="GPU"):
        fn(*args)
