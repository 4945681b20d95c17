"""Trainer-side asymmetric W4A16 QAT (QUADS, arXiv 2607.15810, section 3.2).

The learner fake-quantizes its weights with the same NVFP4 operator the
rollout kernels use, and keeps its activations in bf16:

  forward   W_hat = QDQ_W(W),  Y = X W_hat^T                         Eq. (12)
  backward  dL/dW ~= dL/dW_hat (straight-through),  dL/dX = dY W_hat  Eq. (13)

QDQ_W is `quads_nvfp4_weight_qdq` itself: one dynamic fp32 tensor scale per
expert matrix, E4M3 scales over 16-element blocks along K, E2M1 codes with
ties to even -- the call that produces the rollout's NVFP4 weights.  Its bf16
output is the round-to-nearest-even bf16 of the exact decode v * s_b * s_t,
so the learner sees, bit for bit, the bf16 image of the values the rollout's
W4A4 GEMM multiplies (Eq. (16): the weight term of the mismatch vanishes);
where s_t is a power of two the two are the same numbers.

The matrix product of the learner is the trainer's own (torch); only the QDQ
node runs in the library.
"""

import torch

from . import quads_nvfp4_weight_qdq


class WeightQDQ(torch.autograd.Function):
    """W_hat = QDQ_W(W) for bf16 W [E, N, K] or [N, K]; straight-through gradient."""

    @staticmethod
    def forward(ctx, w):
        if w.dtype != torch.bfloat16:
            raise TypeError("QAT master weights are bf16")
        w3 = w.detach().contiguous()
        squeeze = w3.dim() == 2
        if squeeze:
            w3 = w3.unsqueeze(0)
        if w3.dim() != 3:
            raise ValueError("weights must be [N, K] or [E, N, K]")
        _nib, _scale, _ts, dq = quads_nvfp4_weight_qdq(w3.view(torch.int16), want_dq=True)
        out = dq.view(torch.bfloat16)
        return out[0] if squeeze else out

    @staticmethod
    def backward(ctx, grad):
        return grad                                  # Eq. (13): straight through


def weight_qdq(w):
    """QDQ_W(w) with the straight-through gradient (Eq. (12), (13))."""
    return WeightQDQ.apply(w)


def qat_linear(x, w):
    """Learner forward of one projection under W4A16 QAT: x [.., K] bf16, w [N, K] bf16 master.

    Leading dimensions of x are flattened so that torch runs plain 2-D
    products (forward and backward), never batched ones."""
    k = x.shape[-1]
    y = torch.nn.functional.linear(x.reshape(-1, k), weight_qdq(w))
    return y.reshape(*x.shape[:-1], w.shape[0])
