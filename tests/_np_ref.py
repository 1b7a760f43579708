"""numpy-side helpers for tests: exact decoding of storage dtypes with numpy's
own conversions (independent of the generator's and the oracle's bit code)."""
import numpy as np

DT_F32, DT_BF16, DT_F16 = 0, 1, 2


def decode(dtype: int, a: np.ndarray) -> np.ndarray:
    if dtype == DT_F32:
        return np.asarray(a, np.float32).astype(np.float64)
    a = np.asarray(a, np.uint16)
    if dtype == DT_BF16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.view(np.float16).astype(np.float64)


def encode(dtype: int, x) -> np.ndarray:
    """numpy rounding to the storage dtype (fp32 / fp16 via numpy casts; bf16 by
    truncating an fp32 that is already bf16-representable)."""
    x = np.asarray(x, np.float64)
    if dtype == DT_F32:
        return x.astype(np.float32)
    if dtype == DT_F16:
        return x.astype(np.float16).view(np.uint16)
    f = x.astype(np.float32)
    bits = f.view(np.uint32)
    assert np.all((bits & 0xFFFF) == 0), "bf16 encode expects bf16-representable values"
    return (bits >> 16).astype(np.uint16)


def softmax(x: np.ndarray, T: float) -> np.ndarray:
    z = np.exp((x - x.max()) / T)
    return z / z.sum()


def chi2_pvalue(counts: np.ndarray, probs: np.ndarray) -> float:
    """Pearson chi-square goodness of fit, pooling cells with expected count < 5."""
    from scipy import stats
    counts = np.asarray(counts, np.float64)
    n = counts.sum()
    exp = np.asarray(probs, np.float64) * n
    order = np.argsort(exp)
    c, e = counts[order], exp[order]
    pooled_c, pooled_e, acc_c, acc_e = [], [], 0.0, 0.0
    for ci, ei in zip(c, e):
        acc_c += ci
        acc_e += ei
        if acc_e >= 5:
            pooled_c.append(acc_c); pooled_e.append(acc_e); acc_c = acc_e = 0.0
    if acc_e > 0 or acc_c > 0:
        if pooled_e:
            pooled_c[-1] += acc_c; pooled_e[-1] += acc_e
        else:
            pooled_c.append(acc_c); pooled_e.append(acc_e)
    if len(pooled_c) < 2:
        return 1.0
    return float(stats.chisquare(pooled_c, pooled_e).pvalue)
