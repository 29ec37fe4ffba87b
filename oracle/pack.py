"""4-bit per-block, per-channel key quantization with error-bound metadata.

[S] Methodology > Algorithm Components item 4 fixes only that keys are quantized to 4
bits per block and per channel, in the manner of the KIVI key quantizer, and that the
quantized keys give score bounds that hold with certainty.
Reading taken (test infrastructure only; the HIP pack follows the same rules):

* blocks of 32 consecutive tokens, aligned at multiples of 32; only complete
  blocks are packed;
* zero points on a per-block power-of-two grid: with mn_t = min_i k_it (fp16) and
  A = max_t |mn_t|, kappa = 2^(y - 11) where A = f 2^y, f in [0.5, 1) (kappa = 1 and
  all z = 0 when A = 0); z_t = floor(mn_t / kappa), a 12-bit integer in
  [-2048, 2047]; the zero point is kmin_t = kappa z_t <= mn_t (exact in fp64);
* kscale_t = fp16 round-to-nearest-even of the fp64 value (max_i k_it - kmin_t) / 15;
* code c_it = clamp(rint_half_even((k_it - kmin_t) / kscale_t), 0, 15) in fp64, and 0
  when kscale_t = 0;
* dequantized k~_it = kmin_t + kscale_t c_it (exact in fp64);
* kerr_i = smallest fp16 h with h^2 >= R1-sum_t (k_it - k~_it)^2 * (1 + 2^-40), and
  vnorm_i = smallest fp16 h with h^2 >= R1-sum_t v_it^2 * (1 + 2^-40), so that
  kerr_i >= |k_i - k~_i| and vnorm_i >= |v_i| hold exactly.

The integer zero points make the scan's offset term q.kmin an exact integer dot
product once the query is put on its own power-of-two grid (see ``bounds``).

8-bit refinement copy ([S] Methodology > Algorithm Components item 4: candidates get
an 8-bit refinement before any exact 16-bit read; the pages give no format).  Reading
taken: per token, a symmetric 8-bit code of every channel --

* s8_i = fp32 round-to-nearest-even of the fp64 value max_t |k_it| / 127 (0 for a zero
  key);
* k8_it = clamp(rint_half_even(k_it / s8_i), -127, 127) in fp64 (0 when s8_i = 0);
* k~8_it = s8_i * k8_it (exact in fp64);
* kerr8_i = smallest fp16 h with h^2 >= R1-sum_t (k_it - k~8_it)^2 * (1 + 2^-40).

It is read only for candidates, so it costs no scan bandwidth (134 bytes a candidate
against 256 for the exact key row).
"""

import numpy as np

from .canon import PADF, csum128, fp16_sqrt_up

BLOCK = 32


def pack_kv_4bit(K16: np.ndarray, V16: np.ndarray, nblocks: int) -> dict:
    """Pack blocks 0..nblocks-1 of one layer.

    K16, V16: fp16 [H_kv][n_cap][128].  Returns logical arrays:
    codes u8 [H_kv][32*nblocks][128]; z int16 and kscale fp16 [H_kv][nblocks][128];
    kexp int32 [H_kv][nblocks] (kappa = 2^kexp); kerr and vnorm fp16 [H_kv][32*nblocks];
    the 8-bit copy k8 int8 [H_kv][32*nblocks][128], s8 fp32 and kerr8 fp16 [H_kv][32*nblocks].
    """
    H = K16.shape[0]
    ntok = BLOCK * nblocks
    Kb = K16[:, :ntok].astype(np.float64).reshape(H, nblocks, BLOCK, 128)
    mn = Kb.min(axis=2)
    mx = Kb.max(axis=2)
    A = np.abs(mn).max(axis=2)                                # [H][nb]
    _, y = np.frexp(A)
    kexp = np.where(A > 0, y - 11, 0).astype(np.int32)
    kappa = np.ldexp(1.0, kexp)
    z = np.where(A[..., None] > 0, np.floor(mn / kappa[..., None]), 0.0)
    kmin = kappa[..., None] * z                               # exact
    kscale16 = ((mx - kmin) / 15.0).astype(np.float16)
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
    # the 8-bit copy, per token
    amax = np.abs(Kb).max(axis=3)                             # [H][nb][32], fp16 values
    s8 = (amax / 127.0).astype(np.float32)
    s8d = s8.astype(np.float64)
    k8 = np.clip(np.rint(Kb / np.where(s8d > 0, s8d, 1.0)[..., None]), -127.0, 127.0)
    k8 = np.where(s8d[..., None] > 0, k8, 0.0)
    res8 = Kb - s8d[..., None] * k8
    kerr8 = fp16_sqrt_up(csum128(res8 * res8) * (1.0 + PADF)).reshape(H, ntok)
    return {
        "codes": codes.astype(np.uint8).reshape(H, ntok, 128),
        "z": z.astype(np.int16),
        "kexp": kexp,
        "kscale": kscale16,
        "kerr": kerr.astype(np.float16),
        "vnorm": vnorm.astype(np.float16),
        "k8": k8.astype(np.int8).reshape(H, ntok, 128),
        "s8": s8.reshape(H, ntok),
        "kerr8": kerr8.astype(np.float16),
        "nblocks": nblocks,
    }


def zero_points(packed: dict) -> np.ndarray:
    """kmin = 2^kexp * z as fp64 [H][nb][128]."""
    return np.ldexp(1.0, packed["kexp"])[..., None] * packed["z"].astype(np.float64)
