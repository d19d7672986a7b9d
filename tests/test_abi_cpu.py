"""The C ABI without a GPU: the library loads, exports every declared symbol,
and rejects bad arguments before touching HIP (CPU only, no compute calls)."""
import ctypes
import math
import os
import re

import pytest
import torch

from flashattention_output_re_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa_relayout.h")

# Fake, 16-byte aligned device addresses.  Only ever passed in calls that fail
# validation, which returns before any HIP call.
A, B_, C, O, M = 0x10000, 0x20000, 0x30000, 0x40000, 0x50000


def _header():
    with open(HEADER) as f:
        return f.read()


def declared_functions():
    text = re.sub(r"/\*.*?\*/", "", _header(), flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*((?:attn|relayout)_\w+)\s*\(",
                                 text, re.M)))


def declared_status_codes():
    return {name: int(val) for name, val in
            re.findall(r"#define\s+(FA_E\w+|FA_OK)\s+\(?(-?\d+)\)?", _header())}


@pytest.fixture(scope="module")
def lib():
    return binding.load_library()


def test_every_declared_symbol_is_exported(lib):
    """Every function declared in include/*.h is exported and bound, and the
    binding binds nothing else."""
    import glob
    names = set()
    for path in glob.glob(os.path.join(ROOT, "include", "*.h")):
        with open(path) as f:
            text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
        names |= set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, re.M))
    assert names == set(binding.SIGNATURES), sorted(names ^ set(binding.SIGNATURES))
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version_matches_header(lib):
    v = int(re.search(r"#define\s+FA_ABI_VERSION\s+(\d+)", _header()).group(1))
    assert lib.attn_abi_version() == v == binding.attn_abi_version()


def test_status_codes_and_strings(lib):
    codes = declared_status_codes()
    assert {v: k for k, v in codes.items()} == binding.STATUS_NAMES
    seen = set()
    for code in codes.values():
        s = binding.attn_status_string(code)
        assert s and s != "unknown status"
        seen.add(s)
    assert len(seen) == len(codes)
    assert binding.attn_status_string(12345) == "unknown status"


def _relayout(lib, q=A, k=B_, v=C, out=O, Bn=1, H=2, S=256, D=128, P=2, scale=0.1, mask=None):
    return lib.attn_fwd_relayout_async(q, k, v, out, Bn, H, S, D, P, scale, mask, None)


def _plain(lib, q=A, k=B_, v=C, out=O, Bn=1, H=2, S=256, D=128, scale=0.1, mask=None):
    return lib.attn_fwd_plain_async(q, k, v, out, Bn, H, S, D, scale, mask, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(k=None), -1), (dict(v=None), -1), (dict(out=None), -1),
    (dict(Bn=0), -1), (dict(H=0), -1), (dict(S=0), -1), (dict(P=0), -1), (dict(S=-5), -1),
    (dict(scale=math.inf), -1), (dict(scale=math.nan), -1), (dict(scale=-math.inf), -1),
    (dict(scale=2.0 ** 16 * 1.0000001), -1), (dict(scale=-(2.0 ** 17)), -1), (dict(scale=3e38), -1),
    (dict(scale=2.0 ** 64), -1),
    (dict(S=255, P=2), -2), (dict(S=32760, P=16), -2),
    (dict(D=32), -3), (dict(D=96), -3), (dict(D=256), -3), (dict(D=0), -3),
    (dict(q=A + 8), -4), (dict(k=B_ + 2), -4), (dict(v=C + 4), -4), (dict(out=O + 8), -4),
    (dict(mask=M + 4), -4),
    (dict(S=(1 << 23), D=128, P=1), -5),
    (dict(S=(1 << 23) - 256, D=128, P=1), -5),   # tile-padded offsets reach 2^31
    (dict(Bn=1 << 15, H=1 << 15, S=256, P=1), -5),
])
def test_relayout_validation(lib, kw, code):
    assert _relayout(lib, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(out=None), -1), (dict(H=-1), -1), (dict(scale=math.nan), -1),
    (dict(D=100), -3), (dict(out=O + 2), -4), (dict(S=(1 << 23)), -5),
])
def test_plain_validation(lib, kw, code):
    assert _plain(lib, **kw) == code


def _s2s(lib, q=A, k=B_, v=C, out=O, Bn=1, H=2, S=256, D=128, P=2, scale=0.1, mask=None):
    return lib.attn_fwd_slab_to_slab_async(q, k, v, out, Bn, H, S, D, P, scale, mask, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(v=None), -1), (dict(out=None), -1), (dict(Bn=0), -1),
    (dict(scale=math.nan), -1), (dict(S=255, P=2), -2), (dict(D=96), -3),
    (dict(S=256, P=8), -3),            # 32 tokens per slab: a 64-key stage could span three slabs
    (dict(S=126, P=2), -3),
    (dict(k=B_ + 8), -4), (dict(mask=M + 4), -4),
    (dict(Bn=1, H=1 << 10, S=1 << 13, D=128, P=2), -5),     # 2^31 bytes per input tensor
    (dict(S=(1 << 23), D=128, P=1), -5),
])
def test_slab_to_slab_validation(lib, kw, code):
    assert _s2s(lib, **kw) == code


def _copy(lib, plain=A, out=O, Bn=1, H=2, S=256, D=128, P=2):
    return lib.relayout_to_slabs_async(plain, out, Bn, H, S, D, P, None)


@pytest.mark.parametrize("kw,code", [
    (dict(plain=None), -1), (dict(out=None), -1), (dict(Bn=0), -1), (dict(H=-2), -1),
    (dict(S=0), -1), (dict(P=0), -1), (dict(D=96), -3), (dict(D=0), -3),
    (dict(S=255, P=2), -2), (dict(plain=A + 8), -4), (dict(out=O + 4), -4),
    (dict(Bn=1 << 10, H=1 << 10, S=1 << 10, D=128, P=1), -5),
])
def test_relayout_copy_validation(lib, kw, code):
    assert _copy(lib, **kw) == code


def test_blocking_entry_points_validate(lib):
    assert lib.attn_fwd_relayout(None, B_, C, O, 1, 1, 256, 128, 2, 0.1, None) == -1
    assert lib.attn_fwd_relayout(A, B_, C, O, 1, 1, 256, 128, 3, 0.1, None) == -2
    assert lib.attn_fwd_plain(A, B_, C, O, 1, 1, 256, 48, 0.1, None) == -3
    assert lib.relayout_to_slabs(None, O, 1, 1, 256, 128, 2) == -1
    assert lib.relayout_to_slabs(A, O, 1, 1, 256, 128, 3) == -2
    assert lib.attn_fwd_slab_to_slab(A, B_, C, O, 1, 1, 256, 128, 8, 0.1, None) == -3


@pytest.mark.skipif(torch.cuda.is_available(), reason="only meaningful without a GPU")
def test_valid_arguments_without_device_report_no_device(lib):
    assert _relayout(lib) == -7
    assert _plain(lib) == -7
    assert _copy(lib) == -7
    assert _s2s(lib) == -7


@pytest.mark.skipif(torch.cuda.is_available(), reason="only meaningful without a GPU")
def test_largest_scale_passes_validation(lib):
    assert _relayout(lib, scale=2.0 ** 16) == -7
    assert _relayout(lib, scale=-(2.0 ** 16)) == -7
    assert _instr(lib) == -7


def _instr(lib, q=A, k=B_, v=C, out=O, Bn=1, H=2, S=256, D=128, P=2, scale=0.1, mask=None,
           boundary=0, stamps=0x60000, words=None, units=None):
    if words is None:
        words = 64 * Bn * H * ((S + 127) // 128 + 1)
    return lib.attn_fwd_relayout_instrumented_async(q, k, v, out, Bn, H, S, D, P, scale, mask,
                                                    boundary, stamps, words, units, None)


def test_instrumented_stamp_words(lib):
    assert lib.attn_instrumented_stamp_words(1, 5, 32760) == 64 * 5 * (256 + 1)
    assert lib.attn_instrumented_stamp_words(2, 3, 1) == 64 * 6 * 2
    assert lib.attn_instrumented_stamp_words(0, 3, 100) == 0
    assert binding.attn_instrumented_stamp_words(1, 1, 256) == 64 * 3


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(out=None), -1), (dict(S=0), -1), (dict(scale=math.nan), -1),
    (dict(boundary=3), -1), (dict(boundary=-1), -1), (dict(stamps=None), -1),
    (dict(S=255, P=2), -2), (dict(D=64), -3), (dict(scale=-0.1), -3), (dict(scale=0.0), -3),
    (dict(stamps=0x60004), -4), (dict(q=A + 8), -4),
    (dict(words=64 * 2 * 3 - 1), -5), (dict(S=(1 << 23), P=1), -5),
])
def test_instrumented_validation(lib, kw, code):
    assert _instr(lib, **kw) == code


def _ws(lib, q=A, k=B_, v=C, out=O, Bn=1, H=2, S=4096, D=128, P=2, scale=0.1, mask=None,
        ws=0x70000, nbytes=1 << 30, plain=False, s2s=False):
    if plain:
        return lib.attn_fwd_plain_ws_async(q, k, v, out, Bn, H, S, D, scale, mask, ws, nbytes, None)
    if s2s:
        return lib.attn_fwd_slab_to_slab_ws_async(q, k, v, out, Bn, H, S, D, P, scale, mask, ws,
                                                  nbytes, None)
    return lib.attn_fwd_relayout_ws_async(q, k, v, out, Bn, H, S, D, P, scale, mask, ws, nbytes,
                                          None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(out=None), -1), (dict(Bn=0), -1), (dict(scale=math.nan), -1),
    (dict(nbytes=-1), -1), (dict(S=255, P=2), -2), (dict(D=96), -3), (dict(k=B_ + 8), -4),
    (dict(S=(1 << 23), P=1), -5), (dict(plain=True, D=32), -3), (dict(plain=True, v=None), -1),
    (dict(s2s=True, q=None), -1), (dict(s2s=True, S=256, P=8), -3), (dict(s2s=True, S=255, P=2), -2),
    (dict(s2s=True, nbytes=-1), -1), (dict(s2s=True, k=B_ + 8), -4),
])
def test_workspace_entry_validation(lib, kw, code):
    assert _ws(lib, **kw) == code


@pytest.mark.parametrize("args,code", [((0, 1, 256, 128), -1), ((1, 1, 0, 128), -1),
                                       ((1, 1, 256, 96), -3), ((1, 1, 1 << 23, 128), -5)])
def test_workspace_query_validation(lib, args, code):
    assert lib.attn_fwd_workspace_bytes(*args) == code


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(out=None), -1), (dict(S=0), -1), (dict(scale=2.0 ** 70), -1),
    (dict(S=255, P=2), -2), (dict(D=96), -3), (dict(v=C + 4), -4), (dict(S=(1 << 23), P=1), -5),
])
def test_noalloc_validation(lib, kw, code):
    a = dict(q=A, k=B_, v=C, out=O, Bn=1, H=2, S=4096, D=128, P=2, scale=0.1, mask=None)
    a.update(kw)
    assert lib.attn_fwd_relayout_noalloc_async(a["q"], a["k"], a["v"], a["out"], a["Bn"], a["H"],
                                               a["S"], a["D"], a["P"], a["scale"], a["mask"],
                                               None) == code


@pytest.mark.skipif(torch.cuda.is_available(), reason="only meaningful without a GPU")
def test_workspace_entries_without_device_report_no_device(lib):
    assert _ws(lib) == -7
    assert _ws(lib, plain=True) == -7
    assert _ws(lib, s2s=True) == -7
    assert lib.attn_fwd_workspace_bytes(1, 5, 75600, 128) == -7


def test_python_binding_raises(lib):
    with pytest.raises(binding.FaError) as e:
        lib_call = binding.attn_fwd_relayout_async
        lib_call(None, None, None, None, 1, 1, 256, 64, 3, 0.125, stream=0)
    assert e.value.name == "FA_EINVAL"


def test_binding_rejects_wrong_tensors():
    t = torch.zeros((1, 1, 256, 64), dtype=torch.float32)
    with pytest.raises(TypeError):
        binding._check_tensor("q", t, (1, 1, 256, 64))
    tb = t.to(torch.bfloat16)
    with pytest.raises(ValueError):
        binding._check_tensor("q", tb, (1, 1, 256, 64))   # not on a device
