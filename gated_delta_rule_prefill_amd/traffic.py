"""Algorithmic byte / flop counts used to place measured kernels on the MI355X roofline,
and the DeltaLog traffic / capacity model.

Sources: "DeltaLog：延迟物化递归状态以加速线性注意力解码" reading notes, §1.2 (dense decode
arithmetic intensity, about 4 flop per fp32 state element read and written) and §2.5
(Eqs. 8-11: C_state, C_decay, C_entry, T_dense, T_delta, C_log(M); auxiliary capacity).
"""
from dataclasses import dataclass

HBM_PEAK_BPS = 8.0e12          # MI355X HBM3E, published
BF16_MFMA_PEAK = 2.5e15        # dense bf16 matrix peak, published
FP32_VECTOR_PEAK = 157.3e12


def elem_bytes(dtype_code: int) -> int:
    return 4 if dtype_code == 0 else 2


# ------------------------------------------------------------------------------- prefill
def prefill_bytes(total_tokens: int, H: int, dk: int, dv: int, e: int, perkey: bool,
                  n_seqs: int, init_read: bool) -> int:
    """Bytes a prefill must move at minimum: read q, k [T,H,dk], v [T,H,dv] (e bytes each),
    g (fp32, per head or per key channel), beta (fp32); write o [T,H,dv]; write the final
    fp32 state of every sequence (and read the initial one when it is used)."""
    T = total_tokens
    gate = 4 * T * H * (dk if perkey else 1)
    b = T * H * (2 * dk + dv) * e + gate + 4 * T * H + T * H * dv * e
    b += 4 * n_seqs * H * dk * dv * (2 if init_read else 1)
    return int(b)


def prefill_flops(lengths, H: int, dk: int, dv: int, chunk: int) -> float:
    """Flops the chunked method computes, counting only the causal (triangular) parts:
    per token-head  C*(3*dk + 2*dv)  (A and M products, U, W, the in-chunk read M E ...)
    + 6*dk*dv (W S, Q S, K_g^T E)  + C^2/3 (triangular solve), with C = chunk."""
    tok = sum(int(x) for x in lengths)
    C = chunk
    per = C * (3 * dk + 2 * dv) + 6 * dk * dv + C * C / 3.0
    return float(tok * H * per)


# -------------------------------------------------------------------------------- decode
def decode_bytes(B: int, H: int, dk: int, dv: int, e: int, perkey: bool) -> int:
    """Dense decode step: read + write the fp32 state of every (request, head), read q, k, v
    and the gates, write o, read the slot map."""
    state = 4 * B * H * dk * dv
    return int(2 * state + B * H * (2 * dk + dv) * e + B * H * dv * e
               + 4 * B * H * ((dk if perkey else 1) + 1) + 4 * B)


# ---------------------------------------------------------------------- DeltaLog model
@dataclass
class DeltaLogModel:
    B: int
    H: int
    dk: int
    dv: int
    M: int
    d_lambda: int = 1
    p_S: int = 4
    p_K: int = 2
    p_U: int = 4

    @property
    def c_state(self):
        return self.p_S * self.B * self.H * self.dk * self.dv

    @property
    def c_decay(self):
        return 4 * self.B * self.H * self.d_lambda

    @property
    def c_entry(self):
        return self.B * self.H * (self.p_K * self.dk + self.p_U * self.dv + 4 * self.d_lambda)

    def c_log(self):
        M = self.M
        return ((M - 1) / M + (M - 1) / 2.0) * self.c_entry

    def t_dense(self, common: float = 0.0):
        return common + 2 * self.c_state

    def t_delta(self, common: float = 0.0):
        return (common + self.c_state + self.c_state / self.M + self.c_log()
                + 2 * self.c_decay)

    def aux_bytes(self):
        """Resident bytes of the log and the decay accumulator, (M-1)*C_entry + C_decay."""
        return (self.M - 1) * self.c_entry + self.c_decay

    def profitable(self):
        return self.c_state * (1 - 1.0 / self.M) > self.c_log() + 2 * self.c_decay


def spec_bytes(B: int, n_pos: int, H: int, dk: int, dv: int, e: int, perkey: bool) -> int:
    """Verify step of speculative decoding: per (request, head) one fp32 state read and
    n_pos state writes, plus the n_pos tokens' q, k, v, gates and the outputs."""
    state = 4 * dk * dv
    per_tok = (2 * dk + 2 * dv) * e + 4 * (dk if perkey else 1) + 4
    return B * H * (state * (1 + n_pos) + n_pos * per_tok) + 4 * B * n_pos + 4 * B


def fused_bytes(B: int, H: int, d: int, width: int, e: int) -> int:
    """Fused KDA decode step: read + write the fp32 state, read + write the conv window
    (width - 1 inputs per q/k/v channel), read the new inputs, conv weights, gate inputs and
    parameters, write o, read the slot map."""
    CH = 3 * H * d
    return int(2 * 4 * B * H * d * d + 2 * B * CH * (width - 1) * e + B * CH * e
               + CH * width * 4 + 4 * B * H * d + 4 * B * H + 4 * H + 4 * H * d
               + B * H * d * e + 4 * B)

