"""MI355X (gfx950) decode-time quantized mat-vec (MMVQ).

The compute path is the HIP library ``libmmvq.so`` (C ABI declared in
``include/mmvq.h``); ``binding`` marshals arguments to it. ``synth`` holds
the seeded synthetic input generators.
"""
