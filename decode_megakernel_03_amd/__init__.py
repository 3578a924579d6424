"""MI355X (gfx950) persistent decode megakernel.

``decode_megakernel_03_amd.mk`` is the thin ctypes binding over ``libmk.so`` (the C ABI declared in
``include/mk.h``); ``decode_megakernel_03_amd.synth`` draws seeded synthetic inputs. Importing the
package itself loads nothing.
"""
