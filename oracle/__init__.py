"""Float64 CPU oracle for the Gated Delta Rule-2 (GDN-2) operator.

TEST INFRASTRUCTURE ONLY. This package is the slow, plain reference that the
HIP path is checked against. Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import it. The product path
(``delta_rule_recurrent_gdn_amd``) never imports, calls or links anything here,
and this package imports nothing from the product path.

Sources (the web pages on the method; cited by these tags everywhere):

* [README]  "Gated DeltaNet-2: Decoupling Erase and Write in Linear Attention",
            the NVlabs/GatedDeltaNet-2 README: the gate bullet list (erase
            gate, write gate, channel-wise decay, strict generalization) and
            the update-rule paragraph that follows it. The extracted page text
            lacks the update equation; the paragraph places the erase gate on
            the key side (it multiplies k in the erase, b * k) and the write
            gate on the value side (it multiplies v in the write, w * v).
* [WIKI]    the AI-research-wiki summary of the same paper: TL;DR and
            "Key findings" (chunkwise WY algorithm absorbing channel-wise
            decay into asymmetric erase factors).
* [NEWS]    the aiexpert.news article "Gated DeltaNet-2: finer-grained state
            editing for linear attention": method paragraph.
* [ABS]     the arXiv 2605.22791 abstract (paper-index page and its mirror):
            the update read as a fast-weight write, the delta rule removing
            what the state currently returns for a key before writing to it,
            and the reductions to KDA and Gated DeltaNet.

The recurrence implemented, per batch row and head, with S_t a d_k x d_v
matrix (the form fixed from [README] update-rule paragraph and [ABS]):

    S_t = (I - k_t (b_t * k_t)^T) Diag(alpha_t) S_{t-1} + k_t (w_t * v_t)^T
    o_t = S_t^T q_t

with b_t in [0,1]^{d_k} the erase gate, w_t in [0,1]^{d_v} the write gate and
alpha_t = exp(log_alpha_t) the channel-wise decay on the key axis.

Readings of points the pages leave open:
decay is applied before the erase read (the [README] gate list has the erase
gate act on the state after decay); the output
reads the updated state S_t; q is used as given (no scaling, no normalisation);
gates are post-activation values and gradients are taken with respect to them.

Parity status: every function here is pinned by tests in
``tests/test_oracle_pins.py`` (reductions, closed forms, a hand-computed
example, finite differences and exact gradient identities). The choice of
which erase factor carries b (key-side right factor) and the readout from S_t
rest on the fixed statement of the operator and are not separable by any
reduction the pages state; that reading is "parity unpinned" against the
alternative forms.
"""

from .gdn2 import forward, decode_step, backward  # noqa: F401
from .front_end import gates_from_raw, forward_raw, decode_step_raw, backward_raw  # noqa: F401
from .varlen import forward_varlen, backward_varlen, decode_step_slots  # noqa: F401
from .gate_granularity import forward_gates, backward_gates  # noqa: F401
