"""The Python binding checks caller-supplied tensors before it hands bare pointers to the C ABI (which
cannot check buffer sizes): wrong shapes, dtypes, strides or byte counts raise ValueError before any
library call, and host tensors are refused. Runs on the CPU: every call below stops in the checks."""
import pytest
import torch

mq = pytest.importorskip("sparse_precision_grouped_amd")


def _weights(E=4, N=128, K=256):
    u8 = torch.uint8
    return mq.Weights(torch.zeros((E, N, K // 4), dtype=u8), torch.zeros((E, N, K // 16), dtype=u8),
                      torch.zeros((E, N, K // 32), dtype=u8), torch.ones(E), kl=torch.zeros(1, dtype=u8))


def _gemm_args(rows=16, E=4, K=256):
    return dict(q=torch.zeros((rows, K // 2), dtype=torch.uint8), s=torch.zeros((rows, K // 32), dtype=torch.uint8),
                gamma_a=torch.ones(E), offsets=torch.zeros(E + 1, dtype=torch.int32))


def _raises(match, fn, *a, **kw):
    with pytest.raises(ValueError, match=match):
        fn(*a, **kw)


def test_grouped_gemm_checks():
    W = _weights()
    a = _gemm_args()
    _raises("s: shape", mq.moesq_grouped_gemm, W, a["q"], a["s"][:, :4], a["gamma_a"], a["offsets"])
    _raises("q: dtype", mq.moesq_grouped_gemm, W, a["q"].to(torch.int8), a["s"], a["gamma_a"], a["offsets"])
    _raises("q: shape", mq.moesq_grouped_gemm, W, torch.zeros((16, 64), dtype=torch.uint8), a["s"], a["gamma_a"],
            a["offsets"])
    _raises("gamma_a: shape", mq.moesq_grouped_gemm, W, a["q"], a["s"], torch.ones(3), a["offsets"])
    _raises("offsets: shape", mq.moesq_grouped_gemm, W, a["q"], a["s"], a["gamma_a"], a["offsets"][:4])
    # the capacity layout passes counts [E] instead of offsets [E+1]
    _raises("offsets: shape", mq.moesq_grouped_gemm, W, a["q"], a["s"], a["gamma_a"], a["offsets"],
            flags=mq.F_CAPACITY)
    _raises("xk: shape", mq.moesq_grouped_gemm, W, a["q"], a["s"], a["gamma_a"], a["offsets"],
            xk=torch.zeros((16, 128), dtype=torch.float16))
    _raises("y: shape", mq.moesq_grouped_gemm, W, a["q"], a["s"], a["gamma_a"], a["offsets"],
            y=torch.zeros((16, 64)))
    _raises("y: must be contiguous", mq.moesq_grouped_gemm, W, a["q"], a["s"], a["gamma_a"], a["offsets"],
            y=torch.zeros((128, 16)).t())
    _raises("device tensor", mq.moesq_grouped_gemm, W, a["q"], a["s"], a["gamma_a"], a["offsets"])
    _raises("offsets: shape", mq.moesq_dense_grouped_gemm, W, a["q"], a["s"], a["gamma_a"], a["offsets"][:2])


def test_expert_mlp_checks():
    E, H, I = 4, 256, 256
    W13, W2 = _weights(E, 2 * I, H), _weights(E, H, I)
    a = _gemm_args(16, E, H)
    gh = torch.ones(E)
    _raises("gamma_h: shape", mq.moesq_expert_mlp, W13, W2, a["q"], a["s"], a["gamma_a"], torch.ones(E + 1),
            a["offsets"])
    _raises("y: shape", mq.moesq_expert_mlp, W13, W2, a["q"], a["s"], a["gamma_a"], gh, a["offsets"],
            y=torch.zeros((16, H // 2)))
    # a workspace smaller than the call needs (the library's own size query)
    need = mq.moesq_workspace_bytes(mq.WS_MLP, 16, 0, 0, 0, 0, I)
    _raises("workspace: %d bytes, need %d" % (need - 1, need), mq.moesq_expert_mlp, W13, W2, a["q"], a["s"],
            a["gamma_a"], gh, a["offsets"], y=torch.zeros((16, H)), workspace=torch.zeros(need - 1, dtype=torch.uint8))
    need_d = mq.moesq_workspace_bytes(mq.WS_MLP_DUMP, 16, 0, 0, 0, 0, I)
    _raises("need %d" % need_d, mq.moesq_expert_mlp, W13, W2, a["q"], a["s"], a["gamma_a"], gh, a["offsets"],
            y=torch.zeros((16, H)), workspace=torch.zeros(need, dtype=torch.uint8), flags=mq.F_DUMP_H)
    _raises("calibration", mq.moesq_expert_mlp, W13, W2, a["q"], a["s"], a["gamma_a"], gh, a["offsets"],
            flags=mq.F_CALIBRATE)
    need_c = mq.moesq_workspace_bytes(mq.WS_MLP_CALIBRATE, 0, 0, E)
    _raises("need %d" % need_c, mq.moesq_calibrate_gamma_h, W13, W2, a["q"], a["s"], a["gamma_a"], a["offsets"],
            workspace=torch.zeros(need_c - 4, dtype=torch.uint8))


def test_combine_checks():
    T, k, H = 8, 2, 64
    y = torch.zeros((T * k, H), dtype=torch.bfloat16)
    sp = torch.zeros(T * k, dtype=torch.int32)
    w = torch.ones((T, k))
    _raises("slot_pos: shape", mq.moesq_unpermute_combine, y, sp[:5], w)
    _raises("slot_pos: dtype", mq.moesq_unpermute_combine, y, sp.long(), w)
    _raises("out: shape", mq.moesq_unpermute_combine, y, sp, w, out=torch.zeros((T, H // 2)))
    _raises("device tensor", mq.moesq_unpermute_combine, y, sp, w)
