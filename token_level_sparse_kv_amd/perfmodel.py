"""Algorithmic byte model of one sparse decode step (what the method must move).

Per step, for B sequences, H_kv KV heads of G query heads, head dim d, scoring
rank r, n cached tokens and budget k (bf16 = 2 bytes, fp32 = 4, int32 = 4; the
scoring cache holds kb bytes per element: 2 for bf16, 1 for FP8 E4M3):
  scan    Kproj rows read once:                 B*H_kv*n*r*kb
  attend  selected K and V rows, read in place: B*H_kv*min(k,n)*d*2*2
  select  idx written:                          B*H_kv*k*4
  q read, out written, M read:                  B*H_q*d*2 each, H_kv*r*d*4
  append  k_new, v_new read; K, V, Kproj rows written (T=1 token per (b, h)):
                                                B*H_kv*(4*d*2 + r*kb)
The fp32 score round trip between scan and select is implementation traffic and
is not counted. The dense step it replaces reads B*H_kv*n*d*2*2 bytes of K and V.
"""
from __future__ import annotations


def step_bytes(B, Hkv, G, d, r, n, k, append_tokens=1, kb=2):
    units = B * Hkv
    terms = {
        "scan_kproj": units * n * r * kb,
        "attend_kv_rows": units * min(k, n) * d * 2 * 2,
        "select_idx": units * k * 4,
        "q": B * Hkv * G * d * 2,
        "out": B * Hkv * G * d * 2,
        "M": Hkv * r * d * 4,
        "append": units * append_tokens * (4 * d * 2 + r * kb),
    }
    terms["total"] = sum(terms.values())
    return terms


def dense_kv_bytes(B, Hkv, d, n):
    return B * Hkv * n * d * 2 * 2


MI355X_HBM_PEAK_GBS = 8000.0
