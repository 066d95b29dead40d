"""GPU: the instrumented build's phase records of the decode scoring kernels.

The "phases" build variant (python -m sparse_attention_token_absorb_amd.build
phases) makes every wave of a decode scoring launch record five clock
readings.  Run in a child process (the binding loads one library per
process): one bf16 and one FP8 launch over 2 x 16384 random rows, whose
records must cover every wave of the grid, be ordered in time (start <= first
tile landed <= stream done <= barrier passed <= end), and name XCCs 0-7.  The
child also checks that the instrumented kernels' top-k sets equal those of a
plain top-k of their own scores (the instrumentation changes no result).
Skipped when the instrumented library has not been built.
"""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from sparse_attention_token_absorb_amd import build as hip_build  # noqa: E402

pytestmark = pytest.mark.gpu

CHILD = r"""
import sys
sys.path.insert(0, sys.argv[1])
import numpy as np
import torch
from sparse_attention_token_absorb_amd import binding as B
B.LIB_PATH = sys.argv[2]
B.lib()
dev = torch.device("cuda:0")
g = torch.Generator(device=dev).manual_seed(21)
Bn, N, r, H, k = 2, 16384, 256, 64, 512
pages = Bn * N // 64
bt = torch.arange(pages, dtype=torch.int32, device=dev).reshape(Bn, N // 64)
lens = torch.full((Bn,), N, dtype=torch.int32, device=dev)
seq = torch.arange(Bn, dtype=torch.int32, device=dev)
pos = torch.full((Bn,), N - 1, dtype=torch.int32, device=dev)
w = torch.rand((Bn, H), generator=g, device=dev)
q = torch.randn((Bn, H, 128), generator=g, device=dev).to(torch.bfloat16)
W = (torch.randn((128, r), generator=g, device=dev) / 16).to(torch.bfloat16)
rows = torch.randn((Bn * N, r), generator=g, device=dev).to(torch.bfloat16)
bfc = B.LatentCache(rows.reshape(pages, 64, r).contiguous(), bt, lens)
f8c = B.LatentCache(torch.zeros((pages, 64, r), dtype=torch.uint8, device=dev), bt, lens,
                    torch.zeros((pages, 64, r // 128), dtype=torch.float32, device=dev))
B.append_latent(f8c, rows, torch.arange(Bn, dtype=torch.int32, device=dev).repeat_interleave(N),
                torch.arange(N, dtype=torch.int32, device=dev).repeat(Bn))
for name, which, cache, qt in (("bf16", B.LI_PHASE_SCORE_DECODE_BF16, bfc, B.absorb_query(q, W)),
                               ("fp8", B.LI_PHASE_SCORE_DECODE_FP8, f8c, B.absorb_query(q, W, fp8=True))):
    B.phase_clear(which)
    out = B.score_topk(cache, seq, pos, N, qt, w, k, keep_scores=True)
    torch.cuda.synchronize()
    rec = B.phase_records(which)
    live = rec[rec[:, 0] != 0]
    grid_waves = int(rec[:, 6].max() + 1) * Bn * 4 if len(live) else 0
    assert len(live) == grid_waves and len(live) > 0, (name, len(live), grid_waves)
    t = live[:, :5].astype(np.int64)
    assert (np.diff(t, axis=1) >= 0).all(), name
    assert ((live[:, 5] >> 32) < 8).all(), name
    sc = out.scores.cpu().numpy()
    idx = out.idx.cpu().numpy()
    for b in range(Bn):
        kth = np.sort(sc[b])[-k]
        got = sc[b][idx[b]]
        assert (got >= kth).all() and len(set(idx[b].tolist())) == k, name
    print(name, "waves", len(live), "span_us", round(float((t[:, 4].max() - t[:, 0].min()) * 0.01), 2), flush=True)
print("OK", flush=True)
"""


def test_phase_records_cover_every_wave_in_order():
    if not os.path.exists(hip_build.LIB_PHASES):
        pytest.skip("instrumented library not built (python -m sparse_attention_token_absorb_amd.build phases)")
    r = subprocess.run([sys.executable, "-c", CHILD, ROOT, hip_build.LIB_PHASES], capture_output=True, text=True,
                       timeout=110)
    print(r.stdout[-2000:], r.stderr[-2000:], flush=True)
    assert r.returncode == 0 and r.stdout.strip().endswith("OK")
