"""moesq_expert_mlp_noalloc (the routed-expert MLP whose intermediate buffers live in the library's static
per-GPU scratch array, for callers that cannot allocate) against moesq_expert_mlp with a caller workspace:
the same kernels on the same inputs, so the outputs must be bit-identical. Two calls in a row on the
same array, the second on a smaller batch (it must not see the first call's rows), on both kernel
families, through the C ABI binding."""
import numpy as np
import pytest
import torch

import gen

pytestmark = pytest.mark.gpu

mq = pytest.importorskip("sparse_precision_grouped_amd")
DEV = "cuda"


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _case(E, H, I, T, k, seed):
    rng = np.random.default_rng(seed)
    w13 = (rng.standard_normal((E, 2 * I, H)) * 0.02).astype(np.float32)
    w2 = (rng.standard_normal((E, H, I)) * 0.02).astype(np.float32)
    x = gen.student_t(seed, gen.act_stream(3), T * H).reshape(T, H)
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    return mq.moesq_compress_weights(_dev(w13)), mq.moesq_compress_weights(_dev(w2)), x, ids


def _run_pair(W13, W2, x, ids, E, flags, y_dtype):
    T, k = ids.shape
    H = x.shape[1]
    xd = _dev(x)
    ga = mq.moesq_global_scale(xd).expand(E).contiguous()
    gh = torch.linspace(20.0, 60.0, E, device=DEV)   # a distinct intermediate scale per expert
    rt, q, s = mq.moesq_route_quantize(_dev(ids), E, xd, ga)
    y_ref, _ = mq.moesq_expert_mlp(W13, W2, q, s, ga, gh, rt["offsets"], y_dtype=y_dtype, flags=flags)
    y = torch.full((T * k, H), float("nan"), dtype=y_dtype, device=DEV)
    mq.moesq_expert_mlp_noalloc(W13, W2, q, s, ga, gh, rt["offsets"], y, flags=flags)
    torch.cuda.synchronize()
    bits = torch.int32 if y_dtype == torch.float32 else torch.int16
    return y.view(bits).cpu().numpy(), y_ref.view(bits).cpu().numpy()


@pytest.mark.parametrize("flags", [0, mq.F_FORCE_DECODE, mq.F_FORCE_PREFILL])
def test_noalloc_mlp_two_calls_match_workspace_call(flags):
    E, H, I = 8, 512, 512
    W13, W2, x, ids = _case(E, H, I, 96, 4, 11)
    print("[case] noalloc MLP flags", flags, "rows", ids.size, flush=True)
    for T, ydt in ((96, torch.float32), (20, torch.bfloat16)):   # the second call is smaller
        got, ref = _run_pair(W13, W2, x[:T], ids[:T], E, flags, ydt)
        assert np.array_equal(got, ref), (T, ydt)


def test_noalloc_mlp_limits_and_flags():
    """Batches whose workspace exceeds the static array, and the dump / calibration flags (their results
    would stay in the array), are refused before anything is launched."""
    E, H, I = 4, 256, 256
    W13, W2, x, ids = _case(E, H, I, 16, 2, 12)
    xd = _dev(x)
    ga = mq.moesq_global_scale(xd).expand(E).contiguous()
    gh = torch.full((E,), 40.0, device=DEV)
    rt, q, s = mq.moesq_route_quantize(_dev(ids), E, xd, ga)
    y = torch.empty((32, H), dtype=torch.float32, device=DEV)
    for fl in (mq.F_DUMP_GATEUP, mq.F_DUMP_H, mq.F_CALIBRATE):
        with pytest.raises(mq.MoesqError) as ei:
            mq.moesq_expert_mlp_noalloc(W13, W2, q, s, ga, gh, rt["offsets"], y, flags=fl)
        assert ei.value.status == mq.ERR_INVALID_ARG
    # the largest batch that fits, and one row more (the second fails on the host: nothing runs)
    lo, hi = 1, 1 << 20   # the largest row count whose workspace fits the array
    while lo < hi:
        mid = (lo + hi + 1) // 2
        lo, hi = (mid, hi) if mq.moesq_workspace_bytes(mq.WS_MLP, mid, 0, E, H, 0, I) <= mq.NOALLOC_SCRATCH_BYTES \
            else (lo, mid - 1)
    fits = lo
    g = torch.Generator(device=DEV).manual_seed(5)
    big_q = torch.randint(0, 256, (fits + 1, H // 2), dtype=torch.uint8, device=DEV, generator=g)
    big_s = torch.full((fits + 1, H // 32), 0x30, dtype=torch.uint8, device=DEV)   # UE4M3 0.5
    big_y = torch.empty((fits + 1, H), dtype=torch.float32, device=DEV)
    off = torch.tensor([0, fits + 1, fits + 1, fits + 1, fits + 1], dtype=torch.int32, device=DEV)
    with pytest.raises(mq.MoesqError) as ei:
        mq.moesq_expert_mlp_noalloc(W13, W2, big_q, big_s, ga, gh, off, big_y)
    assert ei.value.status == mq.ERR_WORKSPACE
    # the largest one runs and matches the workspace call (all rows on expert 0)
    off = torch.tensor([0, fits, fits, fits, fits], dtype=torch.int32, device=DEV)
    y_ref, _ = mq.moesq_expert_mlp(W13, W2, big_q[:fits], big_s[:fits], ga, gh, off, y_dtype=torch.float32)
    mq.moesq_expert_mlp_noalloc(W13, W2, big_q[:fits], big_s[:fits], ga, gh, off, big_y[:fits])
    torch.cuda.synchronize()
    assert np.array_equal(big_y[:fits].cpu().numpy(), y_ref.cpu().numpy())
