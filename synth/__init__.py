"""Seeded synthetic inputs for the byte-level BPE encoder: text corpora and
rank tables.

This package holds no part of the encode method.  It draws random text with a
counter-based generator (SplitMix64), and learns rank tables with a plain BPE
trainer whose pre-tokenizer is the third-party ``regex`` module.  Both the
CPU oracle and the GPU library consume what it produces; neither is imported
here.
"""
