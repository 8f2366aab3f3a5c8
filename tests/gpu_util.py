"""Helpers for the GPU tests: move seeded cases to the device and compare with the oracle."""
import os

import numpy as np

BF16_TOL = (2e-2, 2e-3)   # max-abs, mean-abs against the float64 oracle (bf16 path)
FP8_TOL = (5e-2, 5e-3)    # fp8 path


def need_gpu():
    import pytest
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_decode_paged_02_amd as m
    if not os.path.exists(m.LIBRARY_PATH):
        raise RuntimeError("libmla355.so is not built: the GPU tests never fall back to another path")
    return m


def bf16_dev(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def i32_dev(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x).astype(np.int32)).cuda()


def f32_dev(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def u8_dev(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.uint8)).cuda()


def to_f64(t):
    import torch
    return t.float().cpu().numpy().astype(np.float64) if t.dtype == torch.bfloat16 else \
        t.cpu().numpy().astype(np.float64)


def bits_of(t):
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def decode_on_gpu(m, case, num_partitions=0, table=None, cache=None, out=None):
    dev = {
        "q": bf16_dev(case.q),
        "off": i32_dev(case.input_row_offsets),
        "pt": i32_dev(case.page_table if table is None else table),
        "lens": i32_dev(case.cache_lens),
        "cache": bf16_dev(case.latent_cache if cache is None else cache),
    }
    res = m.decode_paged(dev["q"], dev["off"], dev["pt"], dev["lens"], dev["cache"], case.scale,
                         mask=case.mask, local_window_size=case.window,
                         num_partitions=num_partitions, out=out)
    import torch
    torch.cuda.synchronize()
    return res


def compare(got, want, tol, what=""):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    d = np.abs(got - want)
    mx, mean = float(d.max(initial=0.0)), float(d.mean()) if d.size else 0.0
    print(f"[parity] {what}: max-abs {mx:.3e} mean-abs {mean:.3e}", flush=True)
    assert mx <= tol[0] and mean <= tol[1], f"{what}: max-abs {mx:.3e}, mean-abs {mean:.3e} vs {tol}"
    return mx, mean


def decode_fp8_on_gpu(m, case, num_partitions=0, table=None, out=None):
    """Dense fp8 decode of an fp8 DecodeCase through mla_decode_paged_fp8."""
    import torch
    q_scale = f32_dev(case.q_scale) if case.q_scale is not None else None
    c_scale = f32_dev(case.cache_scale) if case.cache_scale is not None else None
    res = m.decode_paged_fp8(u8_dev(case.q8), q_scale, i32_dev(case.input_row_offsets),
                             i32_dev(case.page_table if table is None else table),
                             i32_dev(case.cache_lens), u8_dev(case.cache8), c_scale, case.scale,
                             mask=case.mask, local_window_size=case.window,
                             num_partitions=num_partitions, out=out)
    torch.cuda.synchronize()
    return res
