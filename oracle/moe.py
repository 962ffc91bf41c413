"""Layout, dispatch and combine written out plainly (test infrastructure only).

Source: [DeepEP-TMA] section "High-Level DeepEP API Usage" -- a dispatch call
takes ``hidden_states`` [T, H], ``topk_idx`` [T, k], ``topk_weights`` [T, k]
and ``num_experts`` E, and returns the expert-grouped output together with a
``handle`` that a later combine consumes.  Section "Asynchronous Copy
Primitives" shows that the receive side is a row-for-row copy of bf16 hidden
rows.  The pages do not define the grouping order or the combine; the
readings taken here are:

* expert segments are laid out for e = 0..E-1, back to back, no padding;
* inside a segment, entries keep the row-major order of ``topk_idx``
  (token ascending, then slot), i.e. a stable counting sort by expert;
* combine of token t is sum_j w[t, j] * y[dest_row[t, j]] in fp32, starting
  at +0.0, j ascending, each product and each sum rounded separately (no
  fused multiply-add), then one round-to-nearest-even to bf16;
* an entry whose expert id is outside [0, E) is not placed: its destination
  is -1, it is not counted, and the status word gets
  ``STATUS_EXPERT_OUT_OF_RANGE``; an expert repeated inside one token's row
  sets ``STATUS_DUPLICATE_EXPERT`` but is still placed (each occurrence is
  its own entry);
* dispatch and combine skip an entry whose destination is outside
  [0, recv_rows).

All loops are plain Python over tokens and slots; numpy only stores rows and
does the element-wise fp32 arithmetic of one row at a time.
"""

import numpy as np

from .bf16 import bf16_to_f32, f32_to_bf16_rne

STATUS_EXPERT_OUT_OF_RANGE = 1
STATUS_DUPLICATE_EXPERT = 2


def layout(topk_idx, num_experts):
    """Stable counting sort of the (token, slot) entries by expert.

    Returns a dict with
      counts    int32 [E]    entries routed to each expert
      offsets   int32 [E+1]  exclusive prefix sum of counts (offsets[E] = total)
      dest_row  int32 [T, k] receive row of each entry (-1 if not placed)
      src_token int32 [T*k]  token of each receive row (-1 beyond offsets[E])
      status    int          OR of the STATUS_* bits
    """
    idx = np.asarray(topk_idx)
    T, k = idx.shape
    E = int(num_experts)
    status = 0

    # pass 1: validate and count
    counts = [0] * E
    for t in range(T):
        seen = []
        for j in range(k):
            e = int(idx[t, j])
            if e < 0 or e >= E:
                status |= STATUS_EXPERT_OUT_OF_RANGE
                continue
            if e in seen:
                status |= STATUS_DUPLICATE_EXPERT
            seen.append(e)
            counts[e] += 1

    # exclusive prefix sum over experts
    offsets = [0] * (E + 1)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]

    # pass 2: place entries, a running cursor per expert keeps token order
    cursor = [0] * E
    dest_row = np.full((T, k), -1, dtype=np.int32)
    src_token = np.full(T * k, -1, dtype=np.int32)
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j])
            if e < 0 or e >= E:
                continue
            r = offsets[e] + cursor[e]
            cursor[e] += 1
            dest_row[t, j] = r
            src_token[r] = t

    return {
        "counts": np.array(counts, dtype=np.int32),
        "offsets": np.array(offsets, dtype=np.int32),
        "dest_row": dest_row,
        "src_token": src_token,
        "status": status,
    }


def dispatch(x, dest_row, recv_rows, recv=None):
    """recv[dest_row[t, j], :] = x[t, :] for every placed entry.

    ``x`` is uint16 [T, H] (bf16 bits).  Rows of ``recv`` that no entry
    targets keep what ``recv`` held (zeros when it is created here).
    """
    x = np.asarray(x, dtype=np.uint16)
    dest_row = np.asarray(dest_row)
    T, H = x.shape
    k = dest_row.shape[1]
    if recv is None:
        recv = np.zeros((recv_rows, H), dtype=np.uint16)
    for t in range(T):
        for j in range(k):
            r = int(dest_row[t, j])
            if 0 <= r < recv_rows:
                recv[r, :] = x[t, :]
    return recv


def combine(y, dest_row, topk_w):
    """out[t] = bf16_rne(sum_j w[t, j] * f32(y[dest_row[t, j]])), j ascending.

    ``y`` is uint16 [R, H] (bf16 bits) in the expert-grouped layout,
    ``topk_w`` float32 [T, k] used exactly as given.
    """
    y = np.asarray(y, dtype=np.uint16)
    dest_row = np.asarray(dest_row)
    w = np.asarray(topk_w, dtype=np.float32)
    R, H = y.shape
    T, k = dest_row.shape
    out = np.empty((T, H), dtype=np.uint16)
    for t in range(T):
        acc = np.zeros(H, dtype=np.float32)  # +0.0
        for j in range(k):
            r = int(dest_row[t, j])
            if not (0 <= r < R):
                continue
            prod = w[t, j] * bf16_to_f32(y[r])  # float32 * float32 -> float32
            acc = acc + prod  # separate rounding, never fused
        out[t] = f32_to_bf16_rne(acc)
    return out


def expert_identity(recv):
    """Identity expert: y = recv."""
    return np.array(recv, dtype=np.uint16, copy=True)


def expert_scale(recv, offsets, scales):
    """Per-expert scalar expert: y[r] = bf16_rne(s_e * f32(recv[r])), e = expert of row r."""
    recv = np.asarray(recv, dtype=np.uint16)
    offsets = np.asarray(offsets)
    s = np.asarray(scales, dtype=np.float32)
    y = np.empty_like(recv)
    E = len(offsets) - 1
    for e in range(E):
        for r in range(int(offsets[e]), int(offsets[e + 1])):
            y[r] = f32_to_bf16_rne(s[e] * bf16_to_f32(recv[r]))
    return y
