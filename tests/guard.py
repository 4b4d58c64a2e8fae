"""Output buffers fenced by guard bands, for GPU tests that check a call writes
nothing outside its outputs and workspace.

A fenced buffer lives in the middle of a larger byte allocation whose every
byte starts as 0xFF (a NaN in both bfloat16 and float32).  After the call the
bands before and after the buffer must still be all 0xFF.  Outputs start
as NaN too, so an element the call forgot to write also shows up.
"""

import torch

PAD = 4096  # bytes of guard on each side (keeps the buffer's alignment)
FILL = 0xFF


class Fenced:
    def __init__(self, shape, dtype, device):
        elem = torch.empty((), dtype=dtype).element_size()
        n = 1
        for s in shape:
            n *= int(s)
        self.nbytes = n * elem
        self.raw = torch.full((self.nbytes + 2 * PAD,), FILL, dtype=torch.uint8, device=device)
        self.tensor = self.raw[PAD:PAD + self.nbytes].view(dtype).view(*shape) if n else \
            torch.empty(shape, dtype=dtype, device=device)

    def bands_intact(self):
        lo = self.raw[:PAD]
        hi = self.raw[PAD + self.nbytes:]
        return bool(torch.all(lo == FILL).item()) and bool(torch.all(hi == FILL).item())


def fenced(shape, dtype, device="cuda:0"):
    return Fenced(shape, dtype, device)
