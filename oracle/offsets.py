"""Split sizes to tensor offsets for the grouped linear.

Test infrastructure (see the package docstring): never used by the product path.

"Activation + GroupedLinear Fusion for MOE and other MOE optimizations"
(Description, "Precomputed Tensor Offsets Optimization"; Greptile Summary;
Important Files Changed) computes tensor offsets from the per-group split
sizes once in the forward and saves ``[split_sizes, base_split_offsets,
split_points, input_tensor_offsets, output_tensor_offsets]`` for the
backward; the output offsets are "sized at" the layer's out_features. The
page does not define them. The plainest reading, taken here:

* ``base[0] = 0``, ``base[g+1] = base[g] + splits[g]`` (G+1 int64 values; the
  rows of group g are ``base[g] .. base[g+1]-1``);
* ``split_points = base[1:G]`` (interior boundaries);
* the tensor offsets are ``base * features`` (element offsets into a flat
  [T, features] tensor) for the input and output feature counts.
"""

import numpy as np


def base_offsets(splits):
    """Exclusive prefix sum of the split sizes, length G+1, int64."""
    s = np.asarray(splits, dtype=np.int64)
    out = np.zeros(len(s) + 1, np.int64)
    for g in range(len(s)):
        out[g + 1] = out[g] + s[g]
    return out


def splits_to_offsets(splits, multipliers):
    """[n, G+1] int64: row i is ``base_offsets(splits) * multipliers[i]``."""
    base = base_offsets(splits)
    return np.stack([base * np.int64(m) for m in multipliers]).astype(np.int64)


def split_points(splits):
    """Interior group boundaries base[1:G]."""
    return base_offsets(splits)[1:-1]
