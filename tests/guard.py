"""Canary-guarded GPU buffers for the parity tests.

A buffer handed to the library sits inside a larger allocation whose
margins hold a fixed pattern; after the call the margins are read back, so a
write past either end of the buffer (a dropped-slot store with a wrong
offset, a partial sum outside its split, a cache frame out of place) fails
the test that caused it.
"""
import numpy as np
import torch

NAN_BF16 = 0x7FC0

GUARD = 4096            # bytes of canary before and after each output buffer
CANARY = 0x5AA5


class Guarded:
    """An output buffer inside a larger allocation whose margins hold a
    canary pattern: a write past either end of the buffer changes them."""

    def __init__(self, shape, dtype=torch.bfloat16, fill=NAN_BF16):
        esz = torch.empty((), dtype=dtype).element_size()
        n = int(np.prod(shape))
        assert (n * esz) % 2 == 0
        g = GUARD // 2
        self.full = torch.full((n * esz // 2 + 2 * g,), CANARY, dtype=torch.int16, device="cuda")
        if isinstance(fill, np.ndarray):      # initial contents, as 16-bit patterns
            self.full[g:g + n * esz // 2] = torch.from_numpy(
                np.ascontiguousarray(fill, dtype=np.uint16).view(np.int16).ravel()).cuda()
        else:
            self.full[g:g + n * esz // 2] = fill
        self.g, self.mid = g, n * esz // 2
        self.t = self.full[g:g + self.mid].view(dtype).view(shape)

    def assert_intact(self, what):
        full = self.full.cpu().numpy().view(np.uint16)
        lo, hi = full[:self.g], full[self.g + self.mid:]
        assert np.all(lo == CANARY) and np.all(hi == CANARY), (
            f"{what}: a write landed outside the buffer "
            f"({int(np.sum(lo != CANARY))} units before, {int(np.sum(hi != CANARY))} after)")
