"""Error bound of fp16 GEMM results with fp32 accumulation, shared by the
GPU parity tests and its host check."""
import numpy as np


def ulp16(x):
    """Spacing of float16 at |x| (2**-24 in the subnormal range)."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -14)))
    return 2.0 ** (e - 10)


def fp32_bound_violations(got, ref, Sabs, K):
    """Mask of outputs with |got - ref| > 2 ulp16(ref) + g/(1-g) * Sabs,
    g = K 2**-24: the a-priori error of K-term fp32 accumulation in any order
    (fp16 x fp16 products are exact in fp32, and each addition rounds at most
    once), plus the fp16 roundings of both results (at most 1.5 ulp of
    ref's).  ref: the correctly rounded product; Sabs: the exact sums of
    |a||b| (the oracle on |A| and |B|)."""
    g = K * 2.0 ** -24
    err = np.abs(np.asarray(got, dtype=np.float64) - np.asarray(ref, dtype=np.float64))
    return err > 2 * ulp16(ref) + g / (1 - g) * Sabs
