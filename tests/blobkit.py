"""Hand assembly of expert blobs for the tests, written directly from the
storage format (include/moe.h): sections gate codes, up codes, down codes,
gate (s,z), up (s,z), down (s,z), each 256-byte aligned; codes lowest bits
first in little-endian 32-bit words; (s,z) words hold bf16 s in the low half
and bf16 z in the high half.  Independent of the oracle and of the
generator."""
import numpy as np


def f32_bits_to_bf16(v):
    """Exact bf16 of values that are exactly representable (asserted)."""
    a = np.asarray(v, dtype=np.float32)
    u = a.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value not exactly representable in bf16"
    return (u >> 16).astype(np.uint16)


def pack_codes(q, bits):
    """q: int array [rows][cols] -> uint32 [rows][cols*bits/32]."""
    q = np.asarray(q, dtype=np.uint64)
    rows, cols = q.shape
    cpw = 32 // bits
    q = q.reshape(rows, cols // cpw, cpw)
    shifts = (np.arange(cpw, dtype=np.uint64) * bits)
    return np.bitwise_or.reduce(q << shifts, axis=2).astype(np.uint32)


def pack_sb(s, z):
    """s, z: float arrays [rows][groups] (exact bf16 values) -> uint32."""
    return f32_bits_to_bf16(s).astype(np.uint32) | (f32_bits_to_bf16(z).astype(np.uint32) << 16)


def align256(n):
    return (n + 255) // 256 * 256


def assemble(H, I, bits, q_gate, q_up, q_down, sb_gate, sb_up, sb_down, group=64):
    """Each q_*: codes [rows][cols]; each sb_*: (s, z) arrays [rows][cols/group]."""
    secs = [pack_codes(q_gate, bits), pack_codes(q_up, bits), pack_codes(q_down, bits),
            pack_sb(*sb_gate), pack_sb(*sb_up), pack_sb(*sb_down)]
    out = bytearray()
    for s in secs:
        b = np.ascontiguousarray(s, dtype='<u4').tobytes()
        out += b
        out += bytes(align256(len(out)) - len(out))
    return np.frombuffer(bytes(out), dtype=np.uint8).copy()


def constant_blob(H, I, bits, q, s, z, group=64):
    """Every matrix with code q, scale s and bias z everywhere."""
    def mats(rows, cols):
        return (np.full((rows, cols), q), (np.full((rows, cols // group), s, np.float32),
                                           np.full((rows, cols // group), z, np.float32)))
    qg, sg = mats(I, H)
    qu, su = mats(I, H)
    qd, sd = mats(H, I)
    return assemble(H, I, bits, qg, qu, qd, sg, su, sd, group)
