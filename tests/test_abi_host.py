"""CPU checks of the C ABI: the library loads without touching a device,
exports every symbol include/mok.h declares, and its pure host queries
(config validation, schedule/context sizing, error codes) behave as the
header states. No compute calls: no GPU here."""
import ctypes as C
import math
import os
import re

import pytest

from mokutil import ROOT

import mixture_experts_layer_build_amd as mok
from mixture_experts_layer_build_amd import _lib

HEADER = os.path.join(ROOT, "include", "mok.h")


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mok_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    names = header_functions()
    assert names, "no declarations found in include/mok.h"
    for n in names:
        assert hasattr(lib, n), f"libmok.so does not export {n}"
    assert set(names) == set(_lib.EXPORTS)


def cfg(**kw):
    base = dict(hidden=2048, intermediate=768, num_experts=128, topk=8, max_tokens=8192,
                shared_intermediate=768, capacity_multiplier=1.0, expert_pad=32)
    base.update(kw)
    return mok.MoKConfig(**base)


def status(c):
    cc = c.c()
    return _lib.load().mok_validate_config(C.byref(cc))


def test_validate_config_contract():
    assert status(cfg()) == _lib.MOK_OK
    assert status(cfg(hidden=100)) == _lib.MOK_ERR_UNSUPPORTED
    assert status(cfg(intermediate=96)) == _lib.MOK_ERR_UNSUPPORTED
    assert status(cfg(shared_intermediate=32)) == _lib.MOK_ERR_UNSUPPORTED
    assert status(cfg(expert_pad=48)) == _lib.MOK_ERR_UNSUPPORTED
    # any positive multiple of 32 is a valid pad, also those that do not
    # divide the GEMM tile height or exceed it
    for pad in (32, 64, 96, 160, 192, 224, 288, 512):
        assert status(cfg(expert_pad=pad)) == _lib.MOK_OK, pad
    assert status(cfg(num_experts=2048)) == _lib.MOK_ERR_UNSUPPORTED
    assert status(cfg(topk=0)) == _lib.MOK_ERR_INVALID_ARGUMENT
    assert status(cfg(max_tokens=0)) == _lib.MOK_ERR_INVALID_ARGUMENT
    assert status(cfg(capacity_multiplier=0.0)) == _lib.MOK_ERR_INVALID_ARGUMENT
    assert status(cfg(capacity_multiplier=float("nan"))) == _lib.MOK_ERR_INVALID_ARGUMENT
    # every operand a kernel reads stays below 2 GiB: token rows (up to 127
    # more in the weight gradients' rounded row counts) of the widest of H, I,
    # I_s and 256 (an expert may receive every token), and one expert's weight
    # matrix
    assert status(cfg(max_tokens=(1 << 30) // 2048 - 128)) == _lib.MOK_OK
    assert status(cfg(max_tokens=(1 << 30) // 2048 - 127)) == _lib.MOK_ERR_UNSUPPORTED
    assert status(cfg(intermediate=65536, max_tokens=(1 << 30) // 65536 - 128)) == _lib.MOK_OK
    assert status(cfg(intermediate=65536, max_tokens=(1 << 30) // 65536 - 127)) == _lib.MOK_ERR_UNSUPPORTED
    assert status(cfg(hidden=128, intermediate=64, shared_intermediate=0, max_tokens=(1 << 22) - 128)) == _lib.MOK_OK
    assert status(cfg(hidden=128, intermediate=64, shared_intermediate=0, max_tokens=(1 << 22) - 127)) == \
        _lib.MOK_ERR_UNSUPPORTED
    assert status(cfg(hidden=65536, intermediate=16384 - 64, max_tokens=8)) == _lib.MOK_OK
    assert status(cfg(hidden=65536, intermediate=16384, max_tokens=8)) == _lib.MOK_ERR_UNSUPPORTED
    assert status(cfg(hidden=65536, intermediate=64, shared_intermediate=16384, max_tokens=8)) == \
        _lib.MOK_ERR_UNSUPPORTED
    bad = cfg().c()
    bad.struct_size = 12
    assert _lib.load().mok_validate_config(C.byref(bad)) == _lib.MOK_ERR_INVALID_ARGUMENT
    assert _lib.load().mok_validate_config(None) == _lib.MOK_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("T,H,I,E,k,Is,mult", [
    (256, 128, 64, 8, 2, 0, 1.0), (8192, 2048, 768, 128, 8, 768, 1.0), (16384, 4096, 1536, 32, 4, 1536, 0.5),
    (32768, 7168, 2048, 32, 8, 2048, 1.0)])
def test_schedule_and_context_sizes(T, H, I, E, k, Is, mult):
    c = cfg(hidden=H, intermediate=I, num_experts=E, topk=k, max_tokens=T, shared_intermediate=Is,
            capacity_multiplier=mult)
    L = mok.schedule_layout(c)
    C_ = min(T, math.ceil(mult * T))
    rows_cap = min(T * k, E * C_) + E * 31
    assert L.rows_cap_max == rows_cap
    assert L.n_mb_max == 1
    # fields are ordered, 256-byte aligned and large enough
    offs = [L.header, L.counts, L.kept, L.offsets, L.mb_offsets, L.row_src, L.slot_row, L.tiles, L.total_bytes]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    assert L.slot_row - L.row_src >= 4 * rows_cap
    assert L.tiles - L.slot_row >= 4 * T * k
    assert mok.schedule_bytes(c) == L.total_bytes
    # "at most a few megabytes" at production shapes
    assert L.total_bytes < 8 << 20
    ctx = mok.context_bytes(c)
    assert ctx >= 3 * 2 * (rows_cap * I + T * Is)


def test_minibatch_layout():
    c = cfg(minibatch_size=2048)
    L = mok.schedule_layout(c)
    assert L.n_mb_max == 4
    assert L.row_src - L.mb_offsets >= 4 * 5 * 128


def test_token_ring_contract_and_scratch():
    # the ring is for inference workspaces, in whole minibatches, with E >= k
    assert status(cfg(macrobatch_size=2048, forward_only=1)) == _lib.MOK_OK
    assert status(cfg(macrobatch_size=2048)) == _lib.MOK_ERR_UNSUPPORTED
    assert status(cfg(macrobatch_size=2048, forward_only=1, minibatch_size=1024)) == _lib.MOK_OK
    assert status(cfg(macrobatch_size=2048, forward_only=1, minibatch_size=1536)) == _lib.MOK_ERR_UNSUPPORTED
    assert status(cfg(macrobatch_size=64, forward_only=1, num_experts=4, topk=8)) == _lib.MOK_ERR_UNSUPPORTED
    assert status(cfg(macrobatch_size=-1, forward_only=1)) == _lib.MOK_ERR_INVALID_ARGUMENT
    assert status(cfg(forward_only=2)) == _lib.MOK_ERR_INVALID_ARGUMENT
    # a size of at least max_tokens is one pass, also for training workspaces
    assert status(cfg(macrobatch_size=8192)) == _lib.MOK_OK
    assert status(cfg(macrobatch_size=100000)) == _lib.MOK_OK
    # the schedule's sub-offsets fall on the macrobatch boundaries
    assert mok.schedule_layout(cfg(macrobatch_size=3000, forward_only=1)).n_mb_max == 3
    assert mok.schedule_layout(cfg(macrobatch_size=2048, forward_only=1, minibatch_size=512)).n_mb_max == 16
    # scratch: an inference workspace drops the backward's regions, and the
    # ring sizes the token-proportional forward scratch for one macrobatch
    big = dict(hidden=7168, intermediate=2048, num_experts=32, topk=8, max_tokens=65536, shared_intermediate=2048)
    train = mok.workspace_bytes(cfg(**big))
    infer = mok.workspace_bytes(cfg(forward_only=1, **big))
    ring = mok.workspace_bytes(cfg(forward_only=1, macrobatch_size=8192, **big))
    ring_small = mok.workspace_bytes(cfg(forward_only=1, macrobatch_size=2048, **big))
    assert ring_small < ring < infer / 4 < train / 4
    # h + y + quantized x/h of one 8192-token pass, plus the whole batch's
    # schedule-sized pieces: about an eighth of the one-pass inference scratch
    assert ring < infer * 0.15


def test_invalid_configs_report_zero_sizes_and_raise():
    with pytest.raises(mok.MokError):
        mok.schedule_bytes(cfg(hidden=100))
    cc = cfg(hidden=100).c()
    assert _lib.load().mok_workspace_bytes(C.byref(cc)) == 0


def test_status_strings_and_kernel_names():
    lib = _lib.load()
    for s in range(6):
        assert lib.mok_status_string(s).decode().startswith("MOK_")
    assert lib.mok_kernel_name(-1) == b"unknown"
    assert lib.mok_kernel_name(0) == b"sched_count"


def test_quantize_rejects_bad_arguments_before_any_device_work():
    lib = _lib.load()
    fake = C.c_void_p(16)  # never dereferenced: every case fails host-side checks first
    assert lib.mok_mxfp8_quantize(fake, 0, 4, 48, 48, 1, fake, 48, fake, None) == _lib.MOK_ERR_UNSUPPORTED
    assert lib.mok_mxfp8_quantize(fake, 0, 30, 64, 64, 0, fake, 64, fake, None) == _lib.MOK_ERR_UNSUPPORTED
    assert lib.mok_mxfp8_quantize(fake, 0, 4, 64, 32, 1, fake, 64, fake, None) == _lib.MOK_ERR_INVALID_ARGUMENT
    assert lib.mok_mxfp8_quantize(fake, 0, 4, 64, 64, 2, fake, 64, fake, None) == _lib.MOK_ERR_INVALID_ARGUMENT
    assert lib.mok_mxfp8_quantize(None, 0, 4, 64, 64, 1, fake, 64, fake, None) == _lib.MOK_ERR_INVALID_ARGUMENT
    assert lib.mok_mxfp8_quantize(fake, 0, 0, 64, 64, 1, fake, 64, fake, None) == _lib.MOK_OK


def test_hot_path_calls_reject_null_workspace():
    lib = _lib.load()
    assert lib.mok_build_schedule(None, None, 0, None, 0, None) == _lib.MOK_ERR_INVALID_ARGUMENT
    w = _lib.MokWeights()
    assert lib.mok_forward(None, 0, None, 0, None, None, C.byref(w), None, None, 0, None) == \
        _lib.MOK_ERR_INVALID_ARGUMENT
    out = C.c_void_p()
    cc = cfg(hidden=100).c()
    assert lib.mok_workspace_create(C.byref(cc), 0, C.byref(out)) == _lib.MOK_ERR_UNSUPPORTED
    assert out.value is None
    assert lib.mok_workspace_destroy(None) == _lib.MOK_OK
