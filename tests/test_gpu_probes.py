"""Calibration probes run and give plausible figures (launch cost, read ceiling, grid barrier)."""
import pytest
import torch

import decode_megakernel_wave_amd as mk

pytestmark = pytest.mark.gpu


def test_probes_give_plausible_figures():
    launch = mk.mk_probe_launch(200)
    assert 0 < launch["us_per_launch_pipelined"] < 1000
    assert 0 < launch["us_per_launch_round_trip"] < 10000
    buf = torch.ones(256 << 20, dtype=torch.uint8, device="cuda")
    gbs = mk.mk_probe_read(buf, repeats=3)
    assert 100 < gbs < 20000  # a 256 MiB pass may be served partly by the memory-side cache
    us = mk.mk_probe_barrier(200)
    assert 0 < us < 1000


def test_probe_arguments_are_checked():
    buf = torch.ones(1024, dtype=torch.uint8, device="cuda")
    with pytest.raises(mk.MkError) as e:
        mk.mk_probe_read(buf[1:1001], repeats=1)  # not 16-byte aligned and not a multiple of 16
    assert e.value.code == mk.MK_EINVAL
    with pytest.raises(mk.MkError) as e:
        mk.mk_probe_barrier(0)
    assert e.value.code == mk.MK_EINVAL
