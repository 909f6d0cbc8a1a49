"""Host checks of the number-format facts the kernels build their code
conversions on.  Each one is a property of the IEEE-style formats themselves,
checked here with torch's CPU decoders, so a kernel that relies on it only
needs the property, not a table.

* Down rows of the single-token kernel: a masked code byte (0..15 at 4 bits,
  0..3 at 2 bits) read as an fp8 e4m3 bit pattern is exactly the code times a
  power of two: 2^-9 in the OCP form, 2^-10 in the FNUZ form.  Scaling by a
  power of two commutes with fp32 rounding, so sums of such products are the
  integer-code sums times that power, exactly.
* Gate/up rows of the single-token kernel: fp16 0x6400 | q is 1024 + q and
  0x6400 | (q << 4) is 1024 + 16 q for a 4-bit code q (the 10-bit mantissa
  holds both code positions of a byte).
* The grouped GEMM's weight operand: bf16 0x4300 | q is 128 + q for a 4-bit
  code q, and a code one nibble higher would reach the exponent (bf16 keeps 7
  mantissa bits), which is why that operand takes one shift per code pair.
"""
import torch


def _fp8(codes, dtype):
    return torch.tensor(codes, dtype=torch.uint8).view(dtype).double().tolist()


def test_fp8_code_bytes_are_scaled_integers():
    for bits in (4, 2):
        q = list(range(1 << bits))
        assert _fp8(q, torch.float8_e4m3fn) == [c * 2.0 ** -9 for c in q]
        assert _fp8(q, torch.float8_e4m3fnuz) == [c * 2.0 ** -10 for c in q]


def test_fp8_unit_inverse_is_exact():
    # the kernel multiplies the row scale by 1 / (value of code 1)
    for dtype, e in ((torch.float8_e4m3fn, 9), (torch.float8_e4m3fnuz, 10)):
        u = torch.tensor([1], dtype=torch.uint8).view(dtype).float()
        assert (1.0 / u).item() == 2.0 ** e
        s = torch.tensor([0.0137, -3.5, 1e-3], dtype=torch.bfloat16).float()
        q = torch.tensor([7.0, 15.0, 1.0]) * u
        h = torch.tensor([0.731, -1.25, 3.0e2])
        # (s / u) * (q u * h) and s * (q * h) round identically
        assert torch.equal((s * (1.0 / u)) * (q * h), s * ((q / u) * h))


def test_fp16_magic_code_positions():
    for q in range(16):
        lo = torch.tensor([0x6400 | q], dtype=torch.int16).view(torch.float16).item()
        hi = torch.tensor([0x6400 | (q << 4)], dtype=torch.int16).view(torch.float16).item()
        assert lo == 1024 + q
        assert hi == 1024 + 16 * q


def test_bf16_magic_low_code_only():
    for q in range(16):
        v = torch.tensor([0x4300 | q], dtype=torch.int16).view(torch.bfloat16).item()
        assert v == 128 + q
    # a code in the next nibble sets the exponent's lowest bit for q >= 8:
    # the value becomes 256 + 32 (q - 8), not 128 + 16 q (they meet at q = 8)
    for q in range(8, 16):
        v = torch.tensor([0x4300 | (q << 4)], dtype=torch.int16).view(torch.bfloat16).item()
        assert v == 256 + 32 * (q - 8)
        assert (v == 128 + 16 * q) == (q == 8)
