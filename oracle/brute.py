"""Pure-Python brute force of the same definitions, for tiny inputs.

TEST INFRASTRUCTURE. Written independently of oracle.c as a literal reading of
the definition (POPCORNBENCH "Kimi-K2.6" pages l1_p60, l2_p24, l1_p76, opening
turns: PyTorch Conv1d/Conv3d forward with zero padding, then for the fused op
min over depth and softmax over channels). Every output is the sum, over every
(input channel of its group, kernel tap) pair, of weight times input, where an
input coordinate outside the tensor contributes nothing.
"""
import itertools
import math


def out_len(L, k, s, d, p):
    return (L + 2 * p - d * (k - 1) - 1) // s + 1  # Python // is floor division


def conv(x, w, bias, stride, dilation, padding, groups):
    """x, w nested lists / numpy arrays of any rank (spatial rank = ndim - 2)."""
    import numpy as np
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    nd = x.ndim - 2
    N, Cin = x.shape[:2]
    Cout, Cg = w.shape[:2]
    ks = w.shape[2:]
    Ls = x.shape[2:]
    outs = [out_len(Ls[a], ks[a], stride[a], dilation[a], padding[a]) for a in range(nd)]
    y = np.zeros((N, Cout, *outs), dtype=np.float64)
    per_group_out = Cout // groups
    for n in range(N):
        for co in range(Cout):
            g = co // per_group_out
            for o in itertools.product(*[range(v) for v in outs]):
                s = float(bias[co]) if bias is not None else 0.0
                for cc in range(Cg):
                    ci = g * Cg + cc
                    for t in itertools.product(*[range(v) for v in ks]):
                        pos = [o[a] * stride[a] + t[a] * dilation[a] - padding[a] for a in range(nd)]
                        if all(0 <= pos[a] < Ls[a] for a in range(nd)):
                            s += float(w[(co, cc) + t]) * float(x[(n, ci) + tuple(pos)])
                y[(n, co) + o] = s
    return y


def conv_channels_last(x, w, bias, stride, dilation, padding, groups):
    """The same sum with channels-last indexing: x[n, position..., channel] and
    y[n, position..., output channel]; w[co, c', tap...] as in conv."""
    import numpy as np
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    nd = x.ndim - 2
    N, Cin = x.shape[0], x.shape[-1]
    Cout, Cg = w.shape[:2]
    ks = w.shape[2:]
    Ls = x.shape[1:-1]
    outs = [out_len(Ls[a], ks[a], stride[a], dilation[a], padding[a]) for a in range(nd)]
    y = np.zeros((N, *outs, Cout), dtype=np.float64)
    per_group_out = Cout // groups
    for n in range(N):
        for o in itertools.product(*[range(v) for v in outs]):
            for co in range(Cout):
                g = co // per_group_out
                s = float(bias[co]) if bias is not None else 0.0
                for t in itertools.product(*[range(v) for v in ks]):
                    pos = [o[a] * stride[a] + t[a] * dilation[a] - padding[a] for a in range(nd)]
                    if not all(0 <= pos[a] < Ls[a] for a in range(nd)):
                        continue
                    for cc in range(Cg):
                        s += float(w[(co, cc) + t]) * float(x[(n,) + tuple(pos) + (g * Cg + cc,)])
                y[(n,) + o + (co,)] = s
    return y


def conv3d_min_softmax(x, w, bias, stride, dilation, padding, groups, min_dim=2):
    import numpy as np
    y = conv(x, w, bias, stride, dilation, padding, groups)
    m = y.min(axis=min_dim)
    out = np.empty_like(m)
    N, C = m.shape[:2]
    for n in range(N):
        for idx in itertools.product(*[range(v) for v in m.shape[2:]]):
            vals = [m[(n, c) + idx] for c in range(C)]
            mx = max(vals)
            e = [math.exp(v - mx) for v in vals]
            tot = sum(e)
            for c in range(C):
                out[(n, c) + idx] = e[c] / tot
    return out
