"""Helpers of the GPU parity tests: host <-> device copies and guard canaries."""

import numpy as np
import torch

DEV = "cuda:0"


def bf16_dev(a):
    """numpy uint16 (bf16 bits) -> device bfloat16 tensor."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(DEV)


def u8_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(DEV)


def f32_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def host(t):
    """Device tensor -> numpy (bf16 comes back as uint16 bits)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


class Guarded:
    """An output tensor embedded between two 4 KiB guard zones filled with 0xA5."""

    GUARD = 4096

    def __init__(self, shape, dtype):
        n = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
        g = self.GUARD
        self.raw = torch.full((g + n + g,), 0xA5, dtype=torch.uint8, device=DEV)
        self.t = self.raw[g:g + n].view(dtype).view(shape)
        self.n = n

    def intact(self):
        r = self.raw.cpu().numpy()
        return bool(np.all(r[:self.GUARD] == 0xA5) and np.all(r[self.GUARD + self.n:] == 0xA5))


# ---------------------------------------------------------------------------
# Sampled oracle checks of full-size linears (the oracle quantises only the
# row / column bands it needs; each band's quantisation is independent).

def _oracle():
    import oracle
    return oracle


def weight_rows_deq(w, rows):
    """Dequantised rows `rows` of the 128x128-quantised weight w [N, K] -> f64 [len, K]."""
    oracle = _oracle()
    out = np.zeros((len(rows), w.shape[1]))
    for nb in sorted({int(r) // 128 for r in rows}):
        qb, sb = oracle.quant_weight_128x128(w[128 * nb:128 * nb + 128])
        deq = oracle.dequant_blocks(qb, sb)
        for i, r in enumerate(rows):
            if r // 128 == nb:
                out[i] = deq[r - 128 * nb]
    return out


def weight_cols_deq(w, cols):
    """Dequantised columns of the quantised weight w [N, K] -> f64 [N, len]."""
    oracle = _oracle()
    out = np.zeros((w.shape[0], len(cols)))
    for kb in sorted({int(c) // 128 for c in cols}):
        qb, sb = oracle.quant_weight_128x128(np.ascontiguousarray(w[:, 128 * kb:128 * kb + 128]))
        deq = oracle.dequant_blocks(qb, sb)
        for i, c in enumerate(cols):
            if c // 128 == kb:
                out[:, i] = deq[:, c - 128 * kb]
    return out


def act_rows_deq(x, rows, gamma=None, eps=None):
    """Dequantised rows of quant_act_1x128(x) (or of rmsnorm_quant(x, gamma, eps))."""
    oracle = _oracle()
    xs = np.ascontiguousarray(x[rows])
    q, s = oracle.quant_act_1x128(xs) if gamma is None else oracle.rmsnorm_quant(xs, gamma, eps)
    return oracle.dequant_groups(q, s)


def requant_cols_deq(x, cols, gamma=None, eps=None):
    """Dequantised 128x1 requantised columns of x [M, C] (rows of Qt) -> f64 [len, M]."""
    oracle = _oracle()
    M = x.shape[0]
    out = np.zeros((len(cols), M))
    for g in sorted({int(c) // 128 for c in cols}):
        if gamma is None:
            qg, sg = oracle.quant_act_1x128(np.ascontiguousarray(x[:, 128 * g:128 * g + 128]))
        else:  # RMSNorm needs whole rows: quantise all of x once per group (slow; small M only)
            qa, sa = oracle.rmsnorm_quant(x, gamma, eps)
            qg, sg = np.ascontiguousarray(qa[:, 128 * g:128 * g + 128]), np.ascontiguousarray(sa[g:g + 1])
        qt, st = oracle.requant_transpose_128x1(qg, sg)
        deq = oracle.dequant_groups(qt, st)
        for i, c in enumerate(cols):
            if c // 128 == g:
                out[i] = deq[c - 128 * g]
    return out


def check_sampled(y_bf16, ref, what):
    oracle = _oracle()
    r = oracle.check_gemm(y_bf16, ref, rms=float(np.sqrt(np.mean(ref ** 2))))
    assert r["ok"], f"{what}: {r}"
    return r


def grouped_cols(rng, n, count, per_group=8):
    """`count` sampled column indices of [0, n), 8 per randomly chosen 128-group
    (bounds the number of 128-column bands the oracle has to quantise)."""
    groups = n // 128
    g = rng.choice(groups, min(groups, max(1, count // per_group)), replace=False)
    cols = np.concatenate([128 * gi + rng.choice(128, per_group, replace=False) for gi in g])
    return np.sort(cols[:count] if len(cols) >= count else cols)


def linear_fwd_bwd_check(x, w, dy, name, n_rows=48, n_cols=48, seed=0, backward=True):
    """Run quant -> FProp (and quant dY -> DGrad, requant x2 -> WGrad) on the GPU
    through the C ABI at full size; check sampled outputs against the oracle."""
    import quantized_rl_amd as jet
    M, K = x.shape
    N = w.shape[0]
    print(f"[{name}] M={M} K={K} N={N}", flush=True)
    qx, sx = jet.quantize_act_1x128(bf16_dev(x))
    qw, sw = jet.quantize_weight_128x128(bf16_dev(w))
    y = host(jet.gemm_fprop(qx, sx, qw, sw))
    rng = np.random.default_rng(seed)
    rows_m = np.sort(rng.choice(M, min(n_rows, M), replace=False))
    cols_n = grouped_cols(rng, N, n_cols)
    ref = act_rows_deq(x, rows_m) @ weight_rows_deq(w, cols_n).T
    check_sampled(y[np.ix_(rows_m, cols_n)], ref, f"{name} fprop")
    if not backward:
        return
    qdy, sdy = jet.quantize_act_1x128(bf16_dev(dy))
    dx = host(jet.gemm_dgrad(qdy, sdy, qw, sw))
    qxt, sxt = jet.requant_transpose_128x1(qx, sx)
    qdyt, sdyt = jet.requant_transpose_128x1(qdy, sdy)
    dw = host(jet.gemm_wgrad(qdyt, sdyt, qxt, sxt))
    cols_k = grouped_cols(rng, K, n_cols)
    ref = act_rows_deq(dy, rows_m) @ weight_cols_deq(w, cols_k)
    check_sampled(dx[np.ix_(rows_m, cols_k)], ref, f"{name} dgrad")
    ref = requant_cols_deq(dy, cols_n) @ requant_cols_deq(x, cols_k).T
    check_sampled(dw[np.ix_(cols_n, cols_k)], ref, f"{name} wgrad")
