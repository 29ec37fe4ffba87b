"""4-bit per-block, per-channel key quantization with error-bound metadata.

[S] Methodology > Algorithm Components item 4 fixes only "4-bit per-block-per-
channel quantization (as in KIVI)" used to give deterministic score upper bounds.
Reading taken (test infrastructure only; the HIP pack follows the same rules):

* blocks of 32 consecutive tokens, aligned at multiples of 32; only complete
  blocks are packed;
* per block b and channel t: kmin = min_i k_it (an fp16 value, stored exactly),
  kscale = fp16 round-to-nearest-even of the fp64 value (max - min) / 15;
* code c_it = clamp(rint_half_even((k_it - kmin) / kscale), 0, 15) in fp64, and 0
  when kscale = 0;
* dequantized k~_it = kmin + kscale * c_it (exact in fp64);
* kerr_i = smallest fp16 h with h^2 >= R1-sum_t (k_it - k~_it)^2 * (1 + 2^-40), and
  vnorm_i = smallest fp16 h with h^2 >= R1-sum_t v_it^2 * (1 + 2^-40), so that
  kerr_i >= |k_i - k~_i| and vnorm_i >= |v_i| hold exactly.
"""

import numpy as np

from .canon import PADF, csum128, fp16_sqrt_up

BLOCK = 32


def pack_kv_4bit(K16: np.ndarray, V16: np.ndarray, nblocks: int) -> dict:
    """Pack blocks 0..nblocks-1 of one layer.

    K16, V16: fp16 [H_kv][n_cap][128].  Returns logical arrays:
    codes u8 [H_kv][32*nblocks][128], kmin and kscale fp16 [H_kv][nblocks][128],
    kerr and vnorm fp16 [H_kv][32*nblocks].
    """
    H = K16.shape[0]
    ntok = BLOCK * nblocks
    Kb = K16[:, :ntok].astype(np.float64).reshape(H, nblocks, BLOCK, 128)
    kmin = Kb.min(axis=2)
    kmax = Kb.max(axis=2)
    kscale16 = ((kmax - kmin) / 15.0).astype(np.float16)
    ks = kscale16.astype(np.float64)
    num = Kb - kmin[:, :, None, :]
    safe = np.where(ks > 0, ks, 1.0)[:, :, None, :]
    codes = np.clip(np.rint(num / safe), 0.0, 15.0)
    codes = np.where(ks[:, :, None, :] > 0, codes, 0.0)
    ktil = kmin[:, :, None, :] + ks[:, :, None, :] * codes
    res = Kb - ktil
    kerr = fp16_sqrt_up(csum128(res * res) * (1.0 + PADF)).reshape(H, ntok)
    Vd = V16[:, :ntok].astype(np.float64)
    vnorm = fp16_sqrt_up(csum128(Vd * Vd) * (1.0 + PADF))
    return {
        "codes": codes.astype(np.uint8).reshape(H, ntok, 128),
        "kmin": kmin.astype(np.float16),
        "kscale": kscale16,
        "kerr": kerr.astype(np.float16),
        "vnorm": vnorm.astype(np.float16),
        "nblocks": nblocks,
    }
