"""Fill a decode model with the seeded recipe weights directly on the device.

The fp32 weights come from the device generator (synth_dev.hip, the same
definition the host side feeds the oracle with) and are handed to the model's
own quantiser through its public API.  Nothing here computes any part of the
decode step.
"""
import numpy as np

from . import workloads as W
from . import dev_matrix_rows, draft_map, vector, signs


def load_recipe(model, shape, seed, norm_jitter=0.0, chunk_elems=1 << 26):
    import torch
    buf = torch.empty(chunk_elems, dtype=torch.float32, device=model.device)
    sp = model.stream.cuda_stream
    for spec in W.tensor_specs(shape, norm_jitter):
        if spec.fmt in (W.W4, W.I8):
            step = max(1, chunk_elems // spec.cols)
            for r0 in range(0, spec.rows, step):
                n = min(step, spec.rows - r0)
                view = buf[: n * spec.cols].view(n, spec.cols)
                dev_matrix_rows(view.data_ptr(), spec, seed, r0, n, stream_ptr=sp)
                model.quantize_tensor(spec.layer, spec.kind, r0, view)
        elif spec.fmt == W.VEC:
            model.set_vector(spec.layer, spec.kind, vector(spec, seed))
        elif spec.fmt == W.MAP:
            model.set_draft_map(draft_map(shape, seed))
        else:
            model.set_vector(-1, spec.kind, signs(spec.cols, seed, spec.stream).astype(np.float32))
    model.sync()
    del buf
