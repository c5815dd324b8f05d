"""Chi-square p-value with low-expectation bins merged (test helper)."""
import numpy as np
from scipy import stats


def chisq_pvalue(observed, probs):
    """Pearson chi-square of counts against probabilities; bins are merged in
    order of increasing expectation until each merged bin expects >= 5."""
    observed = np.asarray(observed, dtype=np.float64)
    exp = np.asarray(probs, dtype=np.float64) / np.sum(probs) * observed.sum()
    order = np.argsort(exp)
    obs_m, exp_m = [], []
    acc_o = acc_e = 0.0
    for i in order:
        acc_o += observed[i]
        acc_e += exp[i]
        if acc_e >= 5:
            obs_m.append(acc_o)
            exp_m.append(acc_e)
            acc_o = acc_e = 0.0
    if acc_e > 0 or acc_o > 0:
        obs_m[-1] += acc_o
        exp_m[-1] += acc_e
    return stats.chisquare(obs_m, exp_m).pvalue
