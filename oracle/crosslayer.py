"""One decode step with one selection shared by several layers (test infrastructure only).

Cross-layer reuse of one routing index follows the CLSA abstract (page
"HySparse2 ...": one indexer's top-k reused across layers) and the Kascade
abstract (page "CoSA ...": top-k computed in an anchor layer and reused by the
following layers). Readings: the anchor is the first layer of the group; only
the anchor keeps compressed keys, which grow by the windows completed by the
appended token; the selection is recomputed every step with the anchor's new
query; every layer attends with its own query, keys and values over the shared
block sets.
"""
import numpy as np

from .compress import append_compressed_keys
from .select import SelectParams
from .decode import decode_step


def crosslayer_step(layers, Kc_anchor, seq_lens_old, seq_lens_new, p: SelectParams,
                    scale: float, dtype: str, units=None):
    """layers: list of dicts with Q [B,Hq,d], K, V [B,Hkv,T,d] (already holding the
    appended token). Kc_anchor [B, Hkv, NC, d] valid up to seq_lens_old.

    Returns (new Kc_anchor, blocks, [O per layer], [LSE per layer]).
    """
    a = layers[0]
    B, Hkv = a["K"].shape[:2]
    Kc = Kc_anchor.copy()
    for b in range(B):
        for h in range(Hkv):
            upd = append_compressed_keys(a["K"][b, h], Kc[b, h], int(seq_lens_old[b]),
                                         int(seq_lens_new[b]), dtype)
            Kc[b, h, :upd.shape[0]] = upd
    sel = decode_step(a["Q"], a["Q"], a["K"], a["V"], Kc, seq_lens_new, p, scale, units=units)
    outs, lses = [sel["O"]], [sel["LSE"]]
    for lay in layers[1:]:
        r = decode_step(lay["Q"], lay["Q"], lay["K"], lay["V"], None, seq_lens_new, p, scale,
                        units=list(sel["blocks"].keys()), blocks_override=sel["blocks"])
        outs.append(r["O"])
        lses.append(r["LSE"])
    return Kc, sel["blocks"], outs, lses
